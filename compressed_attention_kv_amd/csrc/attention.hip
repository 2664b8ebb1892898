// attention.hip -- core attention of the CSA and HCA paths on gfx950.
//
// [V4-Pro card, Hybrid attention] 128 query heads of dim 512 share one KV
// head (multi-query attention).  CSA attends to the entries the indexer
// selected, HCA to every visible compressed entry [V4 digest, CSA step 3 and
// HCA paragraph]; both add the raw sliding window and a per-head sink logit
// in the softmax denominator, RMS-normalise query heads and KV vectors before
// the dot product, rotate the last r dims of q, k and the output (the output
// back by -t).  K and V are the same normalised, rotated vector.
//
// Design (one workgroup = one query token, all heads, a range of key tiles):
//   * 4 waves; wave w owns heads [32w, 32w+32).  Its normalised, rotated
//     query block Q^_w (32 x D, f16) stays in VGPRs for the whole kernel as
//     the B operand of S^T = K^ Q^_w^T (v_mfma_f32_32x32x16_f16, keys as rows).
//   * A tile is 32 key slots (selected entries, or visible entries, then the
//     window).  All 256 threads gather the tile rows straight from HBM (each
//     wave instruction reads whole 1 KiB rows), RMS-normalise them (wave
//     reductions), rotate them, convert to f16 and write two LDS copies: K^
//     row-major (QK A operand) and V^T (PV B operand), XOR-swizzled so that
//     MFMA operand reads and the writes are bank-conflict free.  Tiles are
//     double-buffered; the next tile's HBM reads are in flight during the
//     current tile's MFMAs.
//   * Softmax in base 2 with a lazily updated running max (the accumulator
//     is rescaled only when a head's max grows by more than 2^8), so P fits
//     f16 and the 32 x D fp32 accumulator per wave is rarely touched by VALU.
//   * S^T's accumulator layout is exactly the A-operand layout of P for
//     O = P V (keys permuted consistently in V^T), so P never leaves VGPRs.
//   * f16 operands: QK-RMSNorm bounds |x| <= sqrt(D) * max|gamma|, so f16's
//     range is safe and its 11-bit significand is 8x finer than bf16's.
//   * Splits over key tiles write (max, sum, O) partials; a combine kernel
//     merges them with the sink.  With one split the epilogue is fused.
#include <type_traits>

#include "cakv_device.hpp"
#include "cakv_internal.hpp"

namespace cakv {

constexpr int TK = 32;  // key slots per tile

template <typename TIn>
struct ActLoad;

template <>
struct ActLoad<bf16_t> {
    typedef u32x4 raw_t;  // 8 elements
    static __device__ __forceinline__ raw_t load(const bf16_t* p) {
        return *reinterpret_cast<const u32x4*>(p);
    }
    static __device__ __forceinline__ raw_t zero() { return raw_t{0u, 0u, 0u, 0u}; }
    static __device__ __forceinline__ void to_f32(const raw_t& r, float v[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_bits_to_f32(r[i] & 0xffffu);
            v[2 * i + 1] = bf16_bits_to_f32(r[i] >> 16);
        }
    }
};

template <>
struct ActLoad<float> {
    struct raw_t {
        f32x4 a, b;
    };
    static __device__ __forceinline__ raw_t load(const float* p) {
        raw_t r;
        r.a = *reinterpret_cast<const f32x4*>(p);
        r.b = *reinterpret_cast<const f32x4*>(p + 4);
        return r;
    }
    static __device__ __forceinline__ raw_t zero() {
        raw_t r;
        r.a = f32x4{0.f, 0.f, 0.f, 0.f};
        r.b = r.a;
        return r;
    }
    static __device__ __forceinline__ void to_f32(const raw_t& r, float v[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = r.a[i];
            v[4 + i] = r.b[i];
        }
    }
};

// Per-query key-slot geometry: slots [0, n_c) are compressed entries
// (selected idx slots, or entries 0..n_vis-1), slots [n_c, n_c + n_w) are the
// window positions p_lo .. t.
struct QueryGeom {
    int64_t b;
    int32_t t;
    int32_t n_vis;
    int32_t n_c;
    int32_t n_w;
    int32_t p_lo;
    int32_t raw0;
};

template <bool SPARSE>
__device__ __forceinline__ QueryGeom query_geom(const AttnArgs& a, int64_t bq) {
    QueryGeom g;
    g.b = bq / a.Q;
    int32_t t = a.q_pos[bq];
    t = t < 0 ? 0 : t;
    g.t = t;
    int64_t nv = t / a.m;
    g.n_vis = (int32_t)(nv < a.N ? nv : a.N);
    g.n_c = SPARSE ? a.K : g.n_vis;
    int32_t lo = t - a.n_win + 1;
    g.p_lo = lo < 0 ? 0 : lo;
    g.n_w = a.n_win > 0 ? t - g.p_lo + 1 : 0;
    g.raw0 = a.raw_pos0[g.b];
    return g;
}

// Source row, position and validity of key slot `slot`.
template <bool SPARSE, typename TIn>
__device__ __forceinline__ const TIn* slot_row(const AttnArgs& a, const QueryGeom& g, int64_t bq,
                                               int slot, int D, int32_t* pos) {
    if (slot < g.n_c) {
        int32_t j = SPARSE ? a.idx[bq * a.K + slot] : slot;
        if (j < 0 || j >= g.n_vis) return nullptr;
        *pos = j * a.m + a.entry_pos_offset;
        return reinterpret_cast<const TIn*>(a.kv_c) + (g.b * a.N + j) * (int64_t)D;
    }
    int s = slot - g.n_c;
    if (s >= g.n_w) return nullptr;
    int32_t p = g.p_lo + s;
    int64_t row = (int64_t)p - g.raw0;
    if (row < 0 || row >= a.R) return nullptr;
    *pos = p;
    return reinterpret_cast<const TIn*>(a.kv_raw) + (g.b * a.R + row) * (int64_t)D;
}

// tile row of loader key `e` (0..7) of key block kb (0..3): the order that
// makes V^T's virtual slot 8*kb+e match the P operand layout
__device__ __forceinline__ int loader_row(int kb, int e) {
    return 16 * (kb >> 1) + 4 * (kb & 1) + (e & 3) + 8 * (e >> 2);
}

// V^T row placement and granule swizzle (rows are 64 bytes: 32 f16 slots)
__device__ __forceinline__ int vt_offset(int dim, int granule) {
    int P = dim ^ ((dim >> 3) & 3);
    int phys = granule ^ ((P >> 2) & 3) ^ ((P >> 5) & 3);
    return P * 64 + phys * 16;
}

// Per-tile row metadata, written two tiles ahead by wave 0.
struct TileMeta {
    uint64_t rowp[TK];  // source row address, 0 for an empty / invalid slot
    int32_t pos[TK];    // rotary position of the row
    uint32_t mask;      // bit rho set when row rho is a valid key
};

typedef __attribute__((address_space(3))) void lds_void;

// Asynchronous 16-byte-per-lane HBM -> LDS load (global_load_lds_dwordx4):
// lane i writes LDS bytes [lds_base + 16 i, +16).  Written as one asm block
// that saves and restores M0 around the load (M0 carries the LDS base; one
// wait state after writing it), so the compiler neither sees an LDS store
// it would have to wait for nor loses its own M0.  There is no register
// output; completion is awaited explicitly (vmcnt) before the data is read.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gptr), "s"(lds_base)
        : "memory");
}

// The thread index laundered through an empty asm statement: address
// arithmetic derived from it cannot be hoisted out of the tile loop, which
// would pin dozens of loop-invariant addresses in VGPRs for the whole loop.
__device__ __forceinline__ int opaque_tid() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Barrier that waits for this wave's LDS traffic only: asynchronous
// HBM->LDS loads of the next tile stay in flight across it.  Signal fences
// keep the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Barrier after which this workgroup's asynchronous tile loads have landed.
__device__ __forceinline__ void barrier_all() {
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int D, bool SPARSE, typename TIn>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mqa_fwd_kernel(const AttnArgs a) {
    constexpr int G = D / 8;                 // 16-byte f16 granules per K^ row
    constexpr int SWZ = (G < 16 ? G : 16) - 1;
    constexpr int KSTEPS = D / 16;           // QK k-steps
    constexpr int DT = D / 32;               // output dim tiles
    constexpr int KH_BYTES = TK * D * 2;
    constexpr int VT_BYTES = D * TK * 2;
    constexpr bool RAW_F32 = sizeof(TIn) == 4;
    constexpr int RAW_BYTES = TK * D * (int)sizeof(TIn);  // landed (raw) tile rows
    constexpr int CS_FLOATS = TK * kMaxRopePairs * 2;
    constexpr int UNITS = TK * D * (int)sizeof(TIn) / 1024;  // 1 KiB load units per tile
    constexpr int RPU = 1024 / (D * (int)sizeof(TIn));       // rows per unit
    constexpr int LPR = 64 / RPU;                            // lanes per row in a unit
    static_assert(UNITS % 4 == 0 && RPU >= 1, "tile geometry");
    typedef ActLoad<TIn> LD;

    // Raw tile rows land (asynchronously, double-buffered) in raw0/raw1; the
    // normalised K^ and V^T tiles are single-buffered.  Distinct LDS objects,
    // so the compiler can tell the asynchronous loads never alias K^ / V^T.
    __shared__ __attribute__((aligned(16))) uint8_t raw0[RAW_BYTES], raw1[RAW_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t khs[KH_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t vts[VT_BYTES];
    __shared__ __attribute__((aligned(16))) float cs0[CS_FLOATS], cs1[CS_FLOATS];
    __shared__ TileMeta meta[4];
    __shared__ float2 qcs[kMaxRopePairs];
    __shared__ double turns[kMaxRopePairs];
    __shared__ float gkv_s[D];
    __shared__ uint32_t redo;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
    const int lane = tid & 63;
    const int lrow = lane & 31;
    const int lh = lane >> 5;
    const int64_t bq = blockIdx.y;
    const int split = blockIdx.x;
    const int H = a.H;
    const int rope_lo = D - a.rope_dims;
    const int n_pairs = a.rope_dims >> 1;

    const QueryGeom g = query_geom<SPARSE>(a, bq);
    const int L = g.n_c + g.n_w;
    const int n_tiles = (L + TK - 1) / TK;
    const int tps = (n_tiles + a.n_splits - 1) / a.n_splits;
    const int tile0 = split * tps;
    const int tile1 = min(n_tiles, tile0 + tps);

    // wave 0: source rows, positions and validity of tile `tile` -> meta[slot]
    auto tile_meta = [&](int tile, int slot) __attribute__((always_inline)) {
        if (wave != 0) return;
        const int ol = opaque_tid() & 63;
        int32_t pos = 0;
        const TIn* row = nullptr;
        if (ol < TK && tile < tile1) row = slot_row<SPARSE, TIn>(a, g, bq, tile * TK + ol, D, &pos);
        if (ol < TK) {
            meta[slot].rowp[ol] = reinterpret_cast<uint64_t>(row);
            meta[slot].pos[ol] = pos;
        }
        const uint64_t bal = __ballot(row != nullptr);
        if (ol == 0) meta[slot].mask = (uint32_t)bal;
    };
    // all threads: rotary (cos, sin) of the tile rows -> cst
    auto tile_cs = [&](int mslot, float* cst) __attribute__((always_inline)) {
        const int ot = opaque_tid();
        const int rho = ot >> 3, pg = ot & 7;
        const int32_t pos = meta[mslot].pos[rho];
        for (int i = pg; i < n_pairs; i += 8) {
            float sn, cs;
            sincos_turns((double)pos * turns[i], &sn, &cs);
            cst[2 * (rho * kMaxRopePairs + i)] = cs;
            cst[2 * (rho * kMaxRopePairs + i) + 1] = sn;
        }
    };
    // asynchronous HBM -> LDS copy of the tile's rows (global_load_lds_dwordx4):
    // one contiguous 1 KiB unit per wave instruction, rows in tile order.
    auto tile_load = [&](int mslot, uint8_t* dst) __attribute__((always_inline)) {
        const int ol = opaque_tid() & 63;
#pragma unroll
        for (int u = wave; u < UNITS; u += 4) {
            const int rho = u * RPU + ol / LPR;
            const int p = ol % LPR;
            const uint64_t rp = meta[mslot].rowp[rho];
            const int gsrc = p;
            if (rp) lds_dma16(reinterpret_cast<const uint8_t*>(rp) + 16 * gsrc, (uint32_t)(uintptr_t)(dst + 1024 * u));
        }
    };

    // ---------------------------------------------------------------- prologue
    if (wave == 0 && lane < n_pairs) {
        const double tn = rope_turns(a.rope_base, lane, a.rope_dims);
        turns[lane] = tn;
        float sn, cs;
        sincos_turns((double)g.t * tn, &sn, &cs);
        qcs[lane] = make_float2(cs, sn);
    }
    for (int i = tid; i < D; i += 256) gkv_s[i] = a.gamma_kv ? a.gamma_kv[i] : 1.0f;
    tile_meta(tile0, 0);
    tile_meta(tile0 + 1, 1);
    barrier_all();

    // Q^ = RoPE_t(gamma_q * q / rms(q)); wave w stages its 32 heads as f16 in
    // one of the tile buffers (row = head, granules XOR-swizzled by row)
    static_assert(RAW_BYTES >= KH_BYTES, "query staging needs four 32-head buffers");
    const bool has_heads = 32 * wave < H;
    uint8_t* qstage = wave == 0 ? khs : wave == 1 ? vts : wave == 2 ? raw0 : raw1;
    for (int hh = 0; hh < 32; ++hh) {
        const int head = 32 * wave + hh;  // heads >= H are staged as zeros
        const TIn* qrow = reinterpret_cast<const TIn*>(a.q) + (bq * H + (head < H ? head : 0)) * (int64_t)D;
        float v[8];
        if (lane < G && head < H) LD::to_f32(LD::load(qrow + 8 * lane), v);
        else
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.0f;
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(v[i], v[i], ss);
        ss = wave_sum(ss);
        const float inv = __builtin_amdgcn_rsqf(ss / (float)D + a.rms_eps);
        if (lane < G) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] *= inv * (a.gamma_q ? a.gamma_q[8 * lane + i] : 1.0f);
            if (8 * lane >= rope_lo) {
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const float2 c = qcs[(8 * lane + i - rope_lo) >> 1];
                    const float x0 = v[i], x1 = v[i + 1];
                    v[i] = x0 * c.x - x1 * c.y;
                    v[i + 1] = x0 * c.y + x1 * c.x;
                }
            }
            u32x4 w4 = {pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]), pack_f16x2(v[4], v[5]),
                        pack_f16x2(v[6], v[7])};
            *reinterpret_cast<u32x4*>(qstage + hh * (2 * D) + ((lane ^ (hh & SWZ)) << 4)) = w4;
        }
    }
    barrier_lds();
    f16x8 qf[KSTEPS];
    {
        const uint8_t* qrow = qstage + lrow * (2 * D);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
            qf[s] = *reinterpret_cast<const f16x8*>(qrow + (((2 * s + lh) ^ (lrow & SWZ)) << 4));
    }

    // ---------------------------------------------------------------- tile store
    const int kb = tid / G;  // key block (8 slots)
    const int db = tid % G;  // 8-channel granule
    const bool ld_on = tid < 4 * G;
    // normalise, rotate and convert the landed tile rows in place (bf16) or
    // from the raw buffer (f32); write K^ and V^T
    auto store_tile = [&](int mslot, uint8_t* kh, uint8_t* vt, const uint8_t* rawb, const float* cst) __attribute__((always_inline)) {
        if (!ld_on) return;
        const int ot = opaque_tid();
        const int kb = ot / G, db = ot % G;
        const bool rot = 8 * db >= rope_lo;
        uint32_t hk[8][4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int rho = loader_row(kb, e);
            const bool valid = meta[mslot].rowp[rho] != 0ull;
            uint8_t* kslot = kh + rho * (2 * D) + ((db ^ (rho & SWZ)) << 4);
            float v[8];
            if (valid) {
                if (RAW_F32) {
                    const f32x4 x0 = *reinterpret_cast<const f32x4*>(rawb + rho * (4 * D) + 32 * db);
                    const f32x4 x1 = *reinterpret_cast<const f32x4*>(rawb + rho * (4 * D) + 32 * db + 16);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[i] = x0[i];
                        v[4 + i] = x1[i];
                    }
                } else {
                    const u32x4 r = *reinterpret_cast<const u32x4*>(rawb + rho * (2 * D) + 16 * db);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[2 * i] = bf16_bits_to_f32(r[i] & 0xffffu);
                        v[2 * i + 1] = bf16_bits_to_f32(r[i] >> 16);
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = 0.0f;
            }
            float ss = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(v[i], v[i], ss);
            ss = group_sum<G>(ss);
            const float inv = valid ? __builtin_amdgcn_rsqf(ss / (float)D + a.rms_eps) : 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] *= inv * gkv_s[8 * db + i];
            if (rot) {
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const int pi = (8 * db + i - rope_lo) >> 1;
                    const float c = cst[2 * (rho * kMaxRopePairs + pi)], sn = cst[2 * (rho * kMaxRopePairs + pi) + 1];
                    const float x0 = v[i], x1 = v[i + 1];
                    v[i] = x0 * c - x1 * sn;
                    v[i + 1] = x0 * sn + x1 * c;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) hk[e][i] = pack_f16x2(v[2 * i], v[2 * i + 1]);
            *reinterpret_cast<u32x4*>(kslot) = u32x4{hk[e][0], hk[e][1], hk[e][2], hk[e][3]};
            __builtin_amdgcn_sched_barrier(0);  // one key at a time: bounded register use
        }
        // V^T: channel 8*db+i, virtual slots [8*kb, 8*kb+8) = keys e = 0..7
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int half = i & 1, wd = i >> 1;
            uint32_t o[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t x = hk[2 * p][wd], y = hk[2 * p + 1][wd];
                o[p] = half ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
            }
            *reinterpret_cast<u32x4*>(vt + vt_offset(8 * db + i, kb)) = u32x4{o[0], o[1], o[2], o[3]};
        }
    };

    // ---------------------------------------------------------------- state
    // The accumulator is only ever written by MFMAs (and zero-filled), never
    // by VALU, so it can live in AGPRs.  Softmax reference max m_use is fixed
    // per head at the first finite tile max; P = 2^(l - m_use) stays inside
    // f16's range while l <= m_use + 15.  If a later logit exceeds that, the
    // wave flags itself, keeps tracking the true max m_seen, and the tile
    // loop runs a second pass for the flagged waves with m_use = m_seen
    // (then P <= 1).  Typical inputs never take the second pass.
    f32x16 acc[DT];
    float m_use = -INFINITY, m_seen = -INFINITY, l_run = 0.0f;
    bool flagged = false;  // wave-uniform
    bool active = has_heads;

    // QK, softmax and PV on a stored tile
    auto compute_tile = [&](int mslot, const uint8_t* kh, const uint8_t* vt) __attribute__((always_inline)) {
        if (!active) return;
        const uint32_t mask = meta[mslot].mask;
        // per-lane swizzled LDS offsets of the MFMA operand reads, recomputed
        // per tile (a few VALU ops) instead of being held in VGPRs:
        //   K^ row lrow, granule g = 2s + lh  -> koff[s % 8] + 256 * (s / 8)
        //   V^T row 32*dt + lrow, granule g   -> vrow_off + voff[g ^ (dt % 4)] + 2048 * dt
        const int ol = opaque_tid() & 63;
        const int orow = ol & 31, oh = ol >> 5;
        uint32_t koff[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) koff[s] = ((((2 * s + oh) & SWZ) ^ (orow & SWZ)) | ((2 * s + oh) & ~SWZ)) << 4;
        const int lrp = orow ^ ((orow >> 3) & 3);  // V^T row placement within a 32-row block
        const uint32_t vrow_off = (uint32_t)lrp * 64;
        uint32_t voff[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) voff[x] = (uint32_t)((x ^ ((lrp >> 2) & 3)) << 4);
        f32x16 st;
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = 0.0f;
        const uint8_t* krow = kh + orow * (2 * D);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const f16x8 av = *reinterpret_cast<const f16x8*>(krow + koff[s & 7] + 256 * (s >> 3));
            st = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, qf[s], st, 0, 0, 0);
        }
        // softmax numerators for rows 8*(r/4) + 4*lh + r%4 of this tile
        float mx = -INFINITY;
        const uint32_t mrow = mask >> (4 * oh);  // rows 8*(r/4) + 4*oh + r%4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            st[r] = ((mrow >> (8 * (r >> 2) + (r & 3))) & 1u) ? st[r] * a.scale_log2 : -INFINITY;
            mx = fmaxf(mx, st[r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        m_seen = fmaxf(m_seen, mx);
        if (m_use == -INFINITY) m_use = mx;  // nothing accumulated for this head yet
        if (__ballot(mx > m_use + 15.0f)) flagged = true;
        if (flagged) return;
        const bool live = m_use != -INFINITY;
        float psum = 0.0f;
        uint32_t pk[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = live ? __builtin_amdgcn_exp2f(st[r] - m_use) : 0.0f;
            const float p1 = live ? __builtin_amdgcn_exp2f(st[r + 1] - m_use) : 0.0f;
            psum += p0 + p1;
            pk[r >> 1] = pack_f16x2(p0, p1);
        }
        psum += __shfl_xor(psum, 32, 64);
        l_run += psum;
        const f16x8 pa0 = __builtin_bit_cast(f16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
        const f16x8 pa1 = __builtin_bit_cast(f16x8, u32x4{pk[4], pk[5], pk[6], pk[7]});
        const uint8_t* vrow = vt + vrow_off;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f16x8 b0 = *reinterpret_cast<const f16x8*>(vrow + voff[oh ^ (dt & 3)] + 2048 * dt);
            const f16x8 b1 = *reinterpret_cast<const f16x8*>(vrow + voff[(2 + oh) ^ (dt & 3)] + 2048 * dt);
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa0, b0, acc[dt], 0, 0, 0);
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa1, b1, acc[dt], 0, 0, 0);
        }
    };

    // one pipeline step on raw buffer B: store tile `tile` from raw B into
    // K^ / V^T, start loading tile+1 into the other raw buffer, then compute
    auto step = [&](auto bsel, int tile, int it) __attribute__((always_inline)) {
        constexpr int B = decltype(bsel)::value;
        uint8_t* rawc = B == 0 ? raw0 : raw1;
        uint8_t* rawn = B == 0 ? raw1 : raw0;
        float* csc = B == 0 ? cs0 : cs1;
        float* csn = B == 0 ? cs1 : cs0;
        asm volatile("; tile step on buffer set %0" ::"n"(B));  // keeps the two bodies distinct
        store_tile(it & 3, khs, vts, rawc, csc);
        tile_meta(tile + 2, (it + 2) & 3);  // (its index loads complete before the tile loads start)
        if (tile + 1 < tile1) {
            tile_load((it + 1) & 3, rawn);
            tile_cs((it + 1) & 3, csn);
        }
        barrier_lds();
        asm volatile("; compute on buffer set %0" ::"n"(B));
        compute_tile(it & 3, khs, vts);
        barrier_all();
    };

    barrier_lds();  // every wave has read its Q^ block: the buffers are free
    for (int pass = 0; pass < 2; ++pass) {
        active = has_heads && (pass == 0 || flagged);
        if (pass == 1) {
            if (flagged) {
                m_use = m_seen;
                l_run = 0.0f;
                flagged = false;
            }
            tile_meta(tile0, 0);
            tile_meta(tile0 + 1, 1);
            barrier_lds();
        }
        if (active) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;
        }
        if (tile0 < tile1) {
            tile_load(0, raw0);
            tile_cs(0, cs0);
        }
        barrier_all();
        for (int tile = tile0, it = 0; tile < tile1; tile += 2, it += 2) {
            step(std::integral_constant<int, 0>(), tile, it);
            if (tile + 1 < tile1) step(std::integral_constant<int, 1>(), tile + 1, it + 1);
        }
        // does any wave need the second pass?
        if (tid == 0) redo = 0u;
        barrier_lds();
        if (lane == 0 && flagged) redo = 1u;
        barrier_lds();
        if (redo == 0u) break;
    }
    if (!has_heads) return;

    // ---------------------------------------------------------------- epilogue
    // (max, sum, unnormalised O) of this split; the combine kernel folds in
    // the sink, normalises, rotates back and stores.
    const int head = 32 * wave + lrow;
    const int S = a.n_splits;
    const int64_t base = (bq * S + split) * (int64_t)H;
    if (lane < 32 && head < H) {
        a.part_ml[(base + head) * 2] = m_use;
        a.part_ml[(base + head) * 2 + 1] = l_run;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int hr = 32 * wave + 8 * (r >> 2) + 4 * lh + (r & 3);
            if (hr < H) a.part_o[(base + hr) * D + 32 * dt + lrow] = acc[dt][r];
        }
}

// Merge split partials: one workgroup per (query, head), one thread per
// channel pair (so the inverse rotation of a pair stays in one thread).
template <int D>
__global__ __launch_bounds__(256) void mqa_combine_kernel(const AttnArgs a) {
    const int64_t bqh = blockIdx.x;
    const int H = a.H;
    const int64_t bq = bqh / H;
    const int h = (int)(bqh % H);
    const int S = a.n_splits;
    const int pr = threadIdx.x;  // pair index
    if (2 * pr >= D) return;
    const float LOG2E = 1.4426950408889634f;
    const float z = a.sinks[h] * LOG2E;
    float M = z;
    for (int s = 0; s < S; ++s) M = fmaxf(M, a.part_ml[((bq * S + s) * H + h) * 2]);
    float o0 = 0.0f, o1 = 0.0f, Z = 0.0f;
    if (M != -INFINITY) {
        Z = __builtin_amdgcn_exp2f(z - M);
        for (int s = 0; s < S; ++s) {
            const int64_t base = (bq * S + s) * H + h;
            const float ms = a.part_ml[base * 2];
            if (ms == -INFINITY) continue;
            const float e = __builtin_amdgcn_exp2f(ms - M);
            Z += e * a.part_ml[base * 2 + 1];
            const float2 ov = *reinterpret_cast<const float2*>(a.part_o + base * D + 2 * pr);
            o0 = __builtin_fmaf(e, ov.x, o0);
            o1 = __builtin_fmaf(e, ov.y, o1);
        }
        o0 /= Z;
        o1 /= Z;
    }
    const int rope_lo = D - a.rope_dims;
    if (2 * pr >= rope_lo) {
        int32_t t = a.q_pos[bq];
        t = t < 0 ? 0 : t;
        float sn, cs;
        sincos_turns(-(double)t * rope_turns(a.rope_base, (2 * pr - rope_lo) >> 1, a.rope_dims), &sn, &cs);
        const float x0 = o0, x1 = o1;
        o0 = x0 * cs - x1 * sn;
        o1 = x0 * sn + x1 * cs;
    }
    const int64_t off = (bq * H + h) * (int64_t)D + 2 * pr;
    if (a.out_f32) {
        *reinterpret_cast<float2*>(reinterpret_cast<float*>(a.out) + off) = make_float2(o0, o1);
    } else {
        reinterpret_cast<uint32_t*>(a.out)[off >> 1] = f32_to_bf16_bits(o0) | (f32_to_bf16_bits(o1) << 16);
    }
    if (pr == 0 && a.lse)
        a.lse[bq * H + h] = (M == -INFINITY) ? -INFINITY : (M + __builtin_log2f(Z)) * 0.6931471805599453f;
}

template <int D, bool SPARSE, typename TIn>
static int launch_one(const AttnArgs& a, int64_t BQ, hipStream_t stream) {
    dim3 grid((unsigned)a.n_splits, (unsigned)BQ);
    hipLaunchKernelGGL((mqa_fwd_kernel<D, SPARSE, TIn>), grid, dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return -4;
    hipLaunchKernelGGL((mqa_combine_kernel<D>), dim3((unsigned)(BQ * a.H)), dim3(D / 2 < 64 ? 64 : D / 2), 0,
                       stream, a);
    if (hipGetLastError() != hipSuccess) return -4;
    return 0;
}

template <int D>
static int launch_d(const AttnArgs& a, int64_t BQ, bool act_f32, hipStream_t stream) {
    const bool sparse = a.idx != nullptr;
    if constexpr (D <= 128) {
        if (act_f32)
            return sparse ? launch_one<D, true, float>(a, BQ, stream) : launch_one<D, false, float>(a, BQ, stream);
    } else {
        if (act_f32) return -2;  // f32 activations: head dims up to 128
    }
    return sparse ? launch_one<D, true, bf16_t>(a, BQ, stream) : launch_one<D, false, bf16_t>(a, BQ, stream);
}

int launch_mqa_fwd(const AttnArgs& a, int64_t BQ, int D, bool act_f32, hipStream_t stream) {
    if (BQ == 0) return 0;
    switch (D) {
        case 128: return launch_d<128>(a, BQ, act_f32, stream);
        case 512: return launch_d<512>(a, BQ, act_f32, stream);
        default: return -2;
    }
}

}  // namespace cakv
