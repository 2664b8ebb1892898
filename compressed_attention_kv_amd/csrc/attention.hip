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
//   * 4 waves, one per SIMD; wave w owns heads [32w, 32w+32).  Its query
//     block Q~_w (32 x D: RMS-normalised, rotated, times the softmax scale
//     and log2 e; bf16) stays in VGPRs as the B operand of S^T = K Q~_w^T
//     (v_mfma_f32_32x32x16_bf16, keys as rows), and its 32 x D fp32 output
//     accumulator stays in AGPRs.
//   * A tile is 32 key slots: selected (or visible) compressed entries, then
//     the window.  Every key row arrives prepared: kv_prepare normalised and
//     rotated it once, when it was written (a key depends only on its own
//     token or entry and position), so rows are used exactly as they land.
//     Rows are copied
//     HBM -> LDS asynchronously (global_load_lds, 1 KiB per wave instruction)
//     three tiles ahead into a ring of four tile buffers; 16-byte granules are
//     XOR-permuted per row so that both the QK reads and the transposed PV
//     reads (ds_read_b64_tr_b16) run near full LDS rate.  The one LDS tile is
//     both the K and the V operand.
//   * Softmax in base 2 against a per-head reference m_use fixed at the first
//     tile's max, so P = 2^(l - m_use) is never rescaled; a head whose logits
//     later exceed m_use + 15 flags its wave, and a second pass recomputes
//     that wave's heads with the true max.  S^T's accumulator layout is the
//     A-operand layout of P for O = P V (keys permuted consistently in the V
//     reads), so P never leaves VGPRs.
//   * f32 activations (head dims up to 128) run the same schedule on f16
//     operands: their rows are rounded to f16 in LDS one step before use.
//   * Splits over key tiles write (max, sum, O/l) partials; a combine kernel
//     merges them with the sink and rotates the output back.
#include "cakv_attn_common.hpp"
#include "cakv_device.hpp"
#include "cakv_internal.hpp"

namespace cakv {

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
    static __device__ __forceinline__ float sumsq(const raw_t& r, float acc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x2_t w2 = word_as_bf16x2(r[i]);
            acc = __builtin_amdgcn_fdot2_f32_bf16(w2, w2, acc, false);
        }
        return acc;
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
    static __device__ __forceinline__ float sumsq(const raw_t& r, float acc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = __builtin_fmaf(r.a[i], r.a[i], acc);
            acc = __builtin_fmaf(r.b[i], r.b[i], acc);
        }
        return acc;
    }
};

// Per-tile row metadata, written four tiles ahead by wave 0.
struct TileMeta {
    uint64_t rowp[TK];  // source row address, 0 for an empty / invalid slot
    uint32_t mask;      // bit rho set when row rho is a valid key
};

typedef __fp16 h4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) h4 lds_h4;

// The thread index laundered through an empty asm statement: address
// arithmetic derived from it cannot be hoisted out of the tile loop, which
// would pin dozens of loop-invariant addresses in VGPRs for the whole loop.
__device__ __forceinline__ int opaque_tid() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Barrier after which this workgroup's asynchronous tile loads have landed.
__device__ __forceinline__ void barrier_all() {
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Barrier after which all but the last N of this wave's vector-memory loads
// (in issue order) have completed, and all of its LDS traffic: with N = the
// loads of the most recently issued tile, everything older has landed.
template <int N>
__device__ __forceinline__ void barrier_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);  // vmcnt(N) expcnt(7) lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// MFMA operand element of the attention kernel: bf16 for bf16 activations
// (prepared key rows are used exactly as they landed), f16 for f32
// activations (rows are normalised first, so their range is bounded and
// f16's finer significand keeps more of the f32 input).
template <bool F16>
struct MmaOp;

template <>
struct MmaOp<false> {
    typedef bf16x8 vec;
    static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16x2(a, b); }
    static __device__ __forceinline__ float lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
    static __device__ __forceinline__ float hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
    static __device__ __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct MmaOp<true> {
    typedef f16x8 vec;
    static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_f16x2(a, b); }
    static __device__ __forceinline__ float lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[0]; }
    static __device__ __forceinline__ float hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[1]; }
    static __device__ __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// FINAL: the launch has one split per query and writes the output itself
// (two instantiations rather than a runtime branch: the final epilogue's
// values would otherwise stay live in scalar registers across the tile loop).
// CS (channel split, H <= 64): wave w owns heads 32 (w & 1) .. +32 and the
// channel half w >> 1: the QK product runs over its 256 channels and the two
// waves of a head block add their partial logits through LDS (both then hold
// the same logits, softmax and P), and the PV product covers its half of the
// output dims.  Each wave then issues half the MFMAs and LDS reads of a tile,
// so all four SIMDs stay busy when only 64 heads exist.
template <int D, bool SPARSE, typename TIn, bool FINAL, bool CS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mqa_fwd_kernel(const AttnArgs a) {
    constexpr int KSTEPS = D / 16;             // QK k-steps of a whole row
    constexpr int DT = D / 32;                 // output dim tiles of a whole row
    constexpr int KW = CS ? KSTEPS / 2 : KSTEPS;  // k-steps of this wave
    constexpr int DW = CS ? DT / 2 : DT;          // output dim tiles of this wave
    constexpr bool RAW_F32 = sizeof(TIn) == 4;
    constexpr int RB = D * (int)sizeof(TIn);   // bytes of one raw row
    constexpr int RPU = 1024 / RB;             // rows per 1 KiB asynchronous-load unit
    constexpr int LPR = 64 / RPU;              // lanes per row in a unit
    // LDS layout of a tile row.  A 1 KiB row (bf16, D = 512) is one load unit;
    // rows are padded to 1088 bytes and, within each row, 16-byte granule g is
    // stored at g ^ a(r) with a(r) = (r >> 2) & 3 (the loading lanes fetch
    // the permuted granule, so the copy stays one contiguous 1 KiB write).
    // Measured on gfx950, this keeps both operand reads near full LDS rate:
    // the QK reads (16 B of one row per lane, 32 rows) and the transposed PV
    // reads (ds_read_b64_tr_b16, 8 rows x 64 B per instruction).  Smaller
    // rows share a unit and stay packed and unpermuted.
    constexpr bool PERM = RPU == 1;
    constexpr int PAD = PERM ? 64 : 0;
    constexpr int RS = RB + PAD;               // ring row stride; the K row is its first 2D bytes
    constexpr int BUF = TK * RS;               // one tile
    constexpr int UNITS = TK * RB / 1024;      // units per tile
    auto gperm = [](int row) __attribute__((always_inline)) { return PERM ? (row >> 2) & 3 : 0; };
    constexpr int NU = UNITS / 4;              // loads per wave per tile
    constexpr int MS = 8;                      // metadata ring slots
    constexpr int CH = D / 64;                 // 8-channel chunks per lane in the row-norm pass
    static_assert(UNITS % 4 == 0 && RPU >= 1 && BUF >= 32 * (2 * D + PAD), "tile geometry");
    static_assert(!CS || (PERM && !RAW_F32), "channel split: bf16 rows of 1 KiB");
    static_assert(NU + 1 < 64, "vmcnt range");
    typedef ActLoad<TIn> LD;
    typedef MmaOp<RAW_F32> OP;
    typedef typename OP::vec opvec;

    // Four tile buffers in a ring: at step it, buffer it%4 holds the tile
    // being multiplied, (it+1)%4 has landed (f32 rows: rounded to f16 here),
    // (it+2)%4 and (it+3)%4 are still landing.
    __shared__ __attribute__((aligned(16))) uint8_t ring[4][BUF];
    __shared__ TileMeta meta[MS];
    __shared__ int32_t idxs[MS][64];  // sparse: entry indices of a tile (lanes >= TK unused)
    __shared__ __attribute__((aligned(16))) float2 qcs[kMaxRopePairs];
    __shared__ __attribute__((aligned(16))) float fq_s[D];   // gamma_q
    __shared__ __attribute__((aligned(16))) float il_s[4][32];  // 1/l of each head (epilogue)
    __shared__ float sink_s[FINAL ? 128 : 1];  // sink logits, log2 units (one-split epilogue)
    __shared__ uint32_t redo;
    // channel split: each wave's partial logits (16 per lane), read by the
    // other wave of its head block
    __shared__ __attribute__((aligned(16))) float xch[CS ? 4 : 1][16][64];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
    const int lane = tid & 63;
    const int lrow = lane & 31;
    const int lh = lane >> 5;
    const int hbk = CS ? (wave & 1) : wave;   // head block: heads 32 hbk .. +32
    const int chalf = CS ? (wave >> 1) : 0;   // channel half (channel split)
    const int cbyte = 512 * chalf;            // its byte offset in a K row (256 bf16 channels)
    const int64_t wg = xcd_order(blockIdx.x + (int64_t)gridDim.x * blockIdx.y, (int64_t)gridDim.x * gridDim.y);
    const int64_t bq = wg / a.n_splits;
    const int split = (int)(wg % a.n_splits);
    const int H = a.H;
    const int rope_lo = D - a.rope_dims;
    const int n_pairs = a.rope_dims >> 1;

    const QueryGeom g = query_geom<SPARSE>(a, bq);
    const int L = g.n_c + g.n_w;
    const int n_tiles = (L + TK - 1) / TK;
    const int tps = (n_tiles + a.n_splits - 1) / a.n_splits;
    const int tile0 = split * tps;
    const int tile1 = min(n_tiles, tile0 + tps);
    CAKV_DCHECK(bq < (int64_t)gridDim.x * gridDim.y && split < a.n_splits);
    // a row of this query that always exists: the source of loads for empty slots
    const uint8_t* spare_row = reinterpret_cast<const uint8_t*>(a.q) + bq * (int64_t)H * RB;

    // wave 0: source rows, positions and validity of tile `tile` -> meta[slot]
    auto tile_meta = [&](int tile, int slot, int32_t j) __attribute__((always_inline)) {
        if (wave != 0) return;
        const int ol = opaque_tid() & 63;
        const TIn* row = nullptr;
        if (ol < TK && tile < tile1) {
            const int sl = tile * TK + ol;
            row = slot_row<TIn>(a, g, sl, SPARSE ? j : sl, D);
        }
        if (ol < TK) meta[slot].rowp[ol] = reinterpret_cast<uint64_t>(row);
        const uint64_t bal = __ballot(row != nullptr);
        if (ol == 0) meta[slot].mask = (uint32_t)bal;
    };
    // wave 0, sparse: asynchronous copy of the entry indices of `tile` into
    // idxs[slot] (lanes past the selection copy a harmless word)
    auto idx_load = [&](int tile, int slot) __attribute__((always_inline)) {
        const int ol = opaque_tid() & 63;
        const int sl = tile * TK + ol;
        const int32_t* src = (ol < TK && sl < g.n_c) ? a.idx + bq * a.K + sl : a.q_pos + bq;
        lds_dma4(src, (uint32_t)(uintptr_t)&idxs[slot][0]);
    };
    // all waves: asynchronous HBM -> LDS copy of the tile's rows in 1 KiB
    // units, NU per wave; empty slots copy the spare row so that every wave
    // always has exactly NU loads per tile in flight
    auto tile_load = [&](int mslot, uint8_t* dst) __attribute__((always_inline)) {
        const int ol = opaque_tid() & 63;
        uint64_t rp[NU];
#pragma unroll
        for (int k = 0; k < NU; ++k) {
            rp[k] = meta[mslot].rowp[(wave + 4 * k) * RPU + ol / LPR];
            if (RPU == 1) {  // one row per unit: the pointer is wave-uniform, keep it in SGPRs
                // (readfirstlane returns int: widen through uint32_t, never sign-extend)
                const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(rp[k] >> 32));
                const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)rp[k]);
                rp[k] = ((uint64_t)hi << 32) | (uint64_t)lo;
            }
        }
#pragma unroll
        for (int k = 0; k < NU; ++k) {
            const int u = wave + 4 * k;
            const uint8_t* src = rp[k] ? reinterpret_cast<const uint8_t*>(rp[k]) : spare_row;
            lds_dma16(src + 16 * ((ol % LPR) ^ gperm(u)), (uint32_t)(uintptr_t)(dst + (RPU == 1 ? u * RS : 1024 * u)));
        }
    };

    // ---------------------------------------------------------------- prologue
    // Wave 0 requests the entry indices of the first five tiles, then all
    // waves request their query rows; while those are in flight wave 1 fills
    // the rotation table and wave 0 turns the indices into the metadata of the
    // first four tiles.  The first three tiles start landing before the query
    // rows are awaited, and Q~ is built while they land.
    const bool has_heads = 32 * hbk < H;
    const int qhead = 32 * hbk + lrow;
    // metadata of the first four tiles and the indices of the fifth (the
    // entry-index loads are all issued before any is used)
    int32_t jst[5];
    auto meta_issue = [&]() __attribute__((always_inline)) {
        if (wave == 0) {
            const int ol = opaque_tid() & 63;
#pragma unroll
            for (int k = 0; k < 5; ++k) {
                const int t = tile0 + k;
                // an unconditional load from a clamped slot; meta_finish keeps
                // it only for a slot of this split's tiles that holds an entry
                jst[k] = (SPARSE && a.K > 0) ? a.idx[bq * a.K + min(t * TK + ol, a.K - 1)] : 0;
            }
        }
    };
    auto jst_kept = [&](int k, int ol) __attribute__((always_inline)) {
        const int t = tile0 + k;
        return (SPARSE && ol < TK && t < tile1 && t * TK + ol < g.n_c) ? jst[k] : 0;
    };
    auto meta_finish = [&]() __attribute__((always_inline)) {
        if (wave == 0) {
            const int ol = opaque_tid() & 63;
#pragma unroll
            for (int k = 0; k < 4; ++k) tile_meta(tile0 + k, k, jst_kept(k, ol));
            if (SPARSE) idxs[4][ol] = jst_kept(4, ol);
        }
    };
    auto meta_start = [&]() __attribute__((always_inline)) {
        meta_issue();
        meta_finish();
    };
    // the first three tiles start landing; T0 is prepared once it has
    auto start_tiles = [&]() __attribute__((always_inline)) {
        if (tile0 < tile1) tile_load(0, ring[0]);
        if (tile0 + 1 < tile1) tile_load(1, ring[1]);
        if (tile0 + 2 < tile1) tile_load(2, ring[2]);
    };
    meta_issue();
    // small parameters are requested before the query rows, so that storing
    // them in LDS does not wait for those (loads complete in issue order)
    const bool has_gq = a.gamma_q != nullptr;
    constexpr int GQ = (D + 255) / 256;
    // Every lane loads (from clamped addresses): loads under a per-lane
    // condition become exec-masked branches, and the compiler then waits for
    // each such load on the spot and for all loads before the first LDS
    // store, which serialises the prologue's memory latencies.  Lanes past
    // the last head load head 0's row; their results are never stored.
    float gq_pre[GQ];
    if (has_gq) {
#pragma unroll
        for (int k = 0; k < GQ; ++k) gq_pre[k] = a.gamma_q[min(tid + 256 * k, D - 1)];
    } else {
#pragma unroll
        for (int k = 0; k < GQ; ++k) gq_pre[k] = 1.0f;
    }
    const float sink_pre = FINAL ? a.sinks[tid < H ? tid : H - 1] : 0.0f;
    typename LD::raw_t qr[KW];  // lane: head qhead, channels 16 (s + KW chalf) + 8 lh + (0..7)
    {
        const TIn* qrow = reinterpret_cast<const TIn*>(a.q) + (bq * H + (qhead < H ? qhead : 0)) * (int64_t)D + 8 * lh +
                          16 * KW * chalf;
#pragma unroll
        for (int s = 0; s < KW; ++s) qr[s] = LD::load(qrow + 16 * s);
    }
    if (wave == 1 && lane < n_pairs) {
        const double tn = rope_turns(a.rope_ratio, lane);
        float sn, cs;
        sincos_turns((double)g.t * tn, &sn, &cs);
        qcs[lane] = make_float2(cs, sn);
    }
#pragma unroll
    for (int k = 0; k < GQ; ++k)
        if (has_gq && tid + 256 * k < D) fq_s[tid + 256 * k] = gq_pre[k];
    if (FINAL && tid < H) sink_s[tid] = sink_pre * 1.4426950408889634f;
    meta_finish();
    barrier_lds();  // metadata, rotation table and gamma_q visible
    start_tiles();
    // the query rows are older than the tile copies just issued
    if (tile0 + 2 < tile1) wait_vm<3 * NU>();
    else if (tile0 + 1 < tile1) wait_vm<2 * NU>();
    else if (tile0 < tile1) wait_vm<NU>();
    else wait_vm<0>();

    // Q~ = RoPE_t(gamma_q * q) in the B-operand layout of the QK MFMAs: lane
    // (head lrow, half lh) holds channels 16 s + 8 lh + (0..7) for k-step s,
    // so a head's sum of squares is this lane's plus lane l ^ 32's.  The
    // head's 1/rms(q) and the softmax scale (times log2 e) multiply its
    // logits instead: invq, per lane (the logits' column is the head).  f16
    // operands (f32 activations) take 1/rms inside Q~ to bound their range.
    opvec qf[KW];
    float invq;
    {
        float ss = 0.0f;
#pragma unroll
        for (int s = 0; s < KW; ++s) ss = LD::sumsq(qr[s], ss);
        ss = xor32_sum(ss);
        if constexpr (CS) {
            // the head's sum of squares over both channel halves: this wave's
            // plus the partner's (addition commutes, so both get the same bits)
            if (lane < 32) il_s[wave][lrow] = ss;
            barrier_lds();
            ss = ss + il_s[wave ^ 2][lrow];
        }
        const float inv = __builtin_amdgcn_rsqf(ss / (float)D + a.rms_eps);
        invq = RAW_F32 ? a.scale_log2 : inv * a.scale_log2;
        const float qs = RAW_F32 ? inv : 1.0f;
#pragma unroll
        for (int sl = 0; sl < KW; ++sl) {
            const int s = sl + KW * chalf;  // k-step of the whole row (uniform)
            const int d0 = 16 * s + 8 * lh;  // this lane's 8-channel chunk
            const bool rot_any = 16 * s + 16 > rope_lo;  // uniform
            if constexpr (!RAW_F32) {
                if (!has_gq && !rot_any) {  // uniform: the bf16 row as it is
                    qf[sl] = __builtin_bit_cast(opvec, qr[sl]);
                    continue;
                }
            }
            float v[8];
            LD::to_f32(qr[sl], v);
            if (has_gq) {
                const f32x4 f0 = *reinterpret_cast<const f32x4*>(&fq_s[d0]);
                const f32x4 f1 = *reinterpret_cast<const f32x4*>(&fq_s[d0 + 4]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] *= qs * f0[i];
                    v[4 + i] *= qs * f1[i];
                }
            } else if (RAW_F32) {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] *= qs;
            }
            // which channels of k-step s rotate is the same for the whole
            // wave (both halves) unless the boundary falls inside the step
            if (16 * s >= rope_lo && (rope_lo & 7) == 0) {  // uniform: four pairs per lane
                const f32x4 c01 = *reinterpret_cast<const f32x4*>(&qcs[(d0 - rope_lo) >> 1]);
                const f32x4 c23 = *reinterpret_cast<const f32x4*>(&qcs[((d0 - rope_lo) >> 1) + 2]);
                const float cs[4] = {c01[0], c01[2], c23[0], c23[2]}, sn[4] = {c01[1], c01[3], c23[1], c23[3]};
#pragma unroll
                for (int pi = 0; pi < 4; ++pi) {
                    const float x0 = v[2 * pi], x1 = v[2 * pi + 1];
                    v[2 * pi] = x0 * cs[pi] - x1 * sn[pi];
                    v[2 * pi + 1] = x0 * sn[pi] + x1 * cs[pi];
                }
            } else if (16 * s + 16 > rope_lo) {  // uniform: the step holding the boundary, pair by pair
#pragma unroll
                for (int pi = 0; pi < 4; ++pi) {
                    const int d = d0 + 2 * pi;
                    const bool rot = d >= rope_lo;  // rope_dims is even: pairs never straddle it
                    const float2 c = qcs[rot ? (d - rope_lo) >> 1 : 0];
                    const float cs = rot ? c.x : 1.0f, sn = rot ? c.y : 0.0f;
                    const float x0 = v[2 * pi], x1 = v[2 * pi + 1];
                    v[2 * pi] = x0 * cs - x1 * sn;
                    v[2 * pi + 1] = x0 * sn + x1 * cs;
                }
            }
            qf[sl] = __builtin_bit_cast(opvec, u32x4{OP::pack(v[0], v[1]), OP::pack(v[2], v[3]),
                                                      OP::pack(v[4], v[5]), OP::pack(v[6], v[7])});
        }
    }

    // ---------------------------------------------------------------- tile prep
    // f32 rows (already prepared) are rounded to f16 in place, their operand
    // type; bf16 rows are used exactly as they landed.  Lane (row = 8 w + l/8,
    // j = l%8) owns the 8-channel chunks j, j+8, ... of its row; every lane of
    // the wave has read its chunks before any of the writes (LDS operations of
    // one wave complete in order).
    auto prep_tile = [&](int mslot, uint8_t* buf) __attribute__((always_inline)) {
        (void)mslot;
        if constexpr (RAW_F32) {
            const int ot = opaque_tid();
            const int ol = ot & 63;
            const int row = 8 * (ot >> 6) + (ol >> 3);
            const int jj = ol & 7;
            uint8_t* rb = buf + row * RS;
            f32x4 x[CH][2];
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                const int c = jj + 8 * k;
                x[k][0] = *reinterpret_cast<const f32x4*>(rb + 32 * c);
                x[k][1] = *reinterpret_cast<const f32x4*>(rb + 32 * c + 16);
            }
#pragma unroll
            for (int k = 0; k < CH; ++k)
                *reinterpret_cast<u32x4*>(rb + 16 * (jj + 8 * k)) =
                    u32x4{OP::pack(x[k][0][0], x[k][0][1]), OP::pack(x[k][0][2], x[k][0][3]),
                          OP::pack(x[k][1][0], x[k][1][1]), OP::pack(x[k][1][2], x[k][1][3])};
        }
    };

    // ---------------------------------------------------------------- state
    // The accumulator is only ever written by MFMAs (and zero-filled), never
    // by VALU, so it can live in AGPRs.  Softmax reference max m_use is fixed
    // per head at the first finite tile max; P = 2^(l - m_use) <= 2^15 while
    // l <= m_use + 15.  If a later logit exceeds that, the wave flags itself,
    // keeps tracking the true max m_seen, and the tile loop runs a second
    // pass for the flagged waves with m_use = m_seen (then P <= 1).  Typical
    // inputs never take the second pass.
    f32x16 acc[DW];
    float m_use = -INFINITY, m_seen = -INFINITY, l_run = 0.0f;
    bool flagged = false;  // wave-uniform
    bool active = has_heads;

    // QK, softmax and PV on a prepared tile.  S^T = K Q~_w^T (keys as rows);
    // the accumulator layout is the A-operand layout of P for O = P V with
    // the tile's keys in the order (4 lh + j, then 8 + 4 lh + j): the V
    // operand is read in that order straight from the row-major tile with
    // ds_read_b64_tr_b16 (in each 16-lane group, lane i receives element
    // i % 4 of the 8-byte chunks addressed by lanes 4k + i / 4, k = 0..3).
    // channel split: add the other channel half's partial logits (the two
    // waves of a head block exchange them through LDS; every wave takes part
    // in the barrier, also one with no work in this step)
    auto exchange = [&](f32x16& st, bool work) __attribute__((always_inline)) {
        if constexpr (CS) {
            const int ol = opaque_tid() & 63;
            if (work) {
#pragma unroll
                for (int r = 0; r < 16; ++r) xch[wave][r][ol] = st[r];
            }
            barrier_lds();
            if (work) {
#pragma unroll
                for (int r = 0; r < 16; ++r) st[r] = st[r] + xch[wave ^ 2][r][ol];
            }
        }
    };

    auto compute_tile = [&](int mslot, const uint8_t* kh) __attribute__((always_inline)) {
        if (!active) {
            f32x16 none;
            exchange(none, false);
            return;
        }
        const uint32_t mask = __builtin_amdgcn_readfirstlane(meta[mslot].mask);
        const int ol = opaque_tid() & 63;
        const int orow = ol & 31, oh = ol >> 5;
        f32x16 st;
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = 0.0f;
        // K row orow, logical granule 2s + oh, stored at (2s + oh) ^ a(orow):
        // k-step s = 2m + j reads byte 64 m + 32 (j ^ (a >> 1)) + 16 (oh ^ (a & 1));
        // a channel half starts 512 bytes in (the permutation keeps the granule's
        // high bits)
        const int ga = gperm(orow);
        const uint8_t* kq0 = kh + orow * RS + cbyte + 16 * (oh ^ (ga & 1)) + 32 * (ga >> 1);
        const uint8_t* kq1 = kh + orow * RS + cbyte + 16 * (oh ^ (ga & 1)) + 32 * ((ga >> 1) ^ 1);
        auto kread = [&](int s) __attribute__((always_inline)) -> opvec {
            return *reinterpret_cast<const opvec*>(((s & 1) ? kq1 : kq0) + 64 * (s >> 1));
        };
        // K operands QPF k-steps ahead of their MFMA, order pinned through
        // scheduling (left alone, the scheduler shortens the prefetch to save
        // registers and every MFMA waits on LDS latency)
        constexpr int QPF = 6;
        opvec kq[QPF];
#pragma unroll
        for (int s = 0; s < QPF; ++s) kq[s] = kread(s);
#pragma unroll
        for (int s = 0; s < KW; ++s) {
            const opvec av = kq[s % QPF];
            if (s + QPF < KW) kq[s % QPF] = kread(s + QPF);
            st = OP::mfma(av, qf[s], st);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, QPF, 2);
#pragma unroll
        for (int s = 0; s + QPF < KW; ++s) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, QPF, 2);
        exchange(st, true);
        // logits in log2 units: the head's 1/rms(q) times the softmax scale
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] *= invq;
        float mx = -INFINITY;
        if (mask != 0xffffffffu) {
            const uint32_t mrow = mask >> (4 * oh);  // rows 8*(r/4) + 4*oh + r%4
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (!((mrow >> (8 * (r >> 2) + (r & 3))) & 1u)) st[r] = -INFINITY;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[r]);
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
            pk[r >> 1] = OP::pack(p0, p1);
        }
        psum += __shfl_xor(psum, 32, 64);
        l_run += psum;
        const opvec pa[2] = {__builtin_bit_cast(opvec, u32x4{pk[0], pk[1], pk[2], pk[3]}),
                             __builtin_bit_cast(opvec, u32x4{pk[4], pk[5], pk[6], pk[7]})};
        // V operand: lane (group q = ol/16, i = ol%16) addresses row
        // 16 ks + 8 hf + 4 (q/2) + i/4, dims 32 dt + 16 (q%2) + 4 (i%4) .. +3
        const int q = ol >> 4, i16 = ol & 15;
        // (logical granule 4 dt + 2 (q%2) + (i%4)/2, stored at granule ^ a(row):
        // only the low two granule bits change, so dt stays an immediate)
        const uint8_t* vrow[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int rr = 8 * hf + 4 * (q >> 1) + (i16 >> 2);
            vrow[hf] = kh + rr * RS + cbyte + 16 * ((2 * (q & 1) + ((i16 & 3) >> 1)) ^ gperm(rr)) + 8 * (i16 & 1);
        }
        // V operands of output tile dt+1 are read while tile dt is multiplied
        auto vread = [&](int dt, int ks) __attribute__((always_inline)) -> opvec {
            const int off = ks * 16 * RS + 64 * dt;
            const h4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4*)const_cast<uint8_t*>(vrow[0] + off));
            const h4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4*)const_cast<uint8_t*>(vrow[1] + off));
            const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
            return __builtin_bit_cast(opvec, u32x4{w0[0], w0[1], w1[0], w1[1]});
        };
        constexpr int VPF = 2;  // output tiles of V operands in flight ahead of the MFMAs
        opvec vb[VPF + 1][2];
#pragma unroll
        for (int d = 0; d < VPF; ++d) {
            vb[d][0] = vread(d, 0);
            vb[d][1] = vread(d, 1);
        }
#pragma unroll
        for (int dt = 0; dt < DW; ++dt) {
            if (dt + VPF < DW) {
                vb[(dt + VPF) % (VPF + 1)][0] = vread(dt + VPF, 0);
                vb[(dt + VPF) % (VPF + 1)][1] = vread(dt + VPF, 1);
            }
            acc[dt] = OP::mfma(pa[0], vb[dt % (VPF + 1)][0], acc[dt]);
            acc[dt] = OP::mfma(pa[1], vb[dt % (VPF + 1)][1], acc[dt]);
        }
        // keep that order through scheduling: the first tiles' reads, then
        // (MFMA, two reads VPF tiles ahead) pairs, then the last MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * VPF, 0);
#pragma unroll
        for (int dt = 0; dt + VPF < DW; ++dt) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * VPF, 0);
    };

    // One pipeline step (tile T = tile0 + it):
    //   wave 0 builds the metadata of T+4 from its indices (landed) and
    //   starts copying the indices of T+5; all waves start copying the rows
    //   of T+3; T+1's f32 rows are rounded to f16 while T is multiplied
    //   (different buffers, no barrier between them); the closing barrier
    //   waits until only T+3's rows are in flight.
    auto step = [&](int it) __attribute__((always_inline)) {
        const int T = tile0 + it;
        if (wave == 0) {
            const int ol = opaque_tid() & 63;
            tile_meta(T + 4, (it + 4) & (MS - 1), SPARSE ? idxs[(it + 4) & (MS - 1)][ol] : 0);
            if (SPARSE && T + 5 < tile1) idx_load(T + 5, (it + 5) & (MS - 1));
        }
        const bool more = T + 3 < tile1;
        if (more) tile_load((it + 3) & (MS - 1), ring[(it + 3) & 3]);
        asm volatile("; prep phase" ::);
        if (T + 1 < tile1) prep_tile((it + 1) & (MS - 1), ring[(it + 1) & 3]);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("; compute phase" ::);
        compute_tile(it & (MS - 1), ring[it & 3]);
        asm volatile("; end of step" ::);
        if (more) barrier_vm<NU>();
        else barrier_vm<0>();
    };

    // Fast step (bf16 1 KiB rows; T a full tile, T+3 inside the split; an
    // active wave that has not flagged): one block in three phases whose VALU
    // work rides under MFMAs (branching only on a pass's first tile).
    //   A: the QK MFMAs of T, with the copy of T+3 between them (one row unit
    //      every four MFMAs);
    //   B: P for the first eight keys of T (P no longer waits on the tile
    //      max: a tile that would flag the wave only spoils a pass that the
    //      second pass redoes);
    //   C: the PV MFMAs of T for k-step 0, then 1, with the other eight
    //      keys' P, the max and the sums between them.
    auto step_fast = [&](int it) __attribute__((always_inline)) {
        const int T = tile0 + it;
        if (wave == 0) {
            const int ol0 = opaque_tid() & 63;
            tile_meta(T + 4, (it + 4) & (MS - 1), SPARSE ? idxs[(it + 4) & (MS - 1)][ol0] : 0);
            if (SPARSE && T + 5 < tile1) idx_load(T + 5, (it + 5) & (MS - 1));
        }
        const int ms3 = (it + 3) & (MS - 1);
        const uint8_t* kh = ring[it & 3];
        uint8_t* db = ring[(it + 3) & 3];
        const int ol = opaque_tid() & 63;
        // row pointers of T+3 (one row per unit: wave-uniform)
        uint64_t rp[NU];
#pragma unroll
        for (int k = 0; k < NU; ++k) {
            const uint64_t v = meta[ms3].rowp[wave + 4 * k];
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
            rp[k] = ((uint64_t)hi << 32) | (uint64_t)lo;
        }
        auto dma_unit = [&](int k) __attribute__((always_inline)) {
            const int u = wave + 4 * k;
            const uint8_t* src = rp[k] ? reinterpret_cast<const uint8_t*>(rp[k]) : spare_row;
            lds_dma16_nc(src + 16 * ((ol % LPR) ^ gperm(u)), (uint32_t)(uintptr_t)(db + u * RS));
        };
        // ---- A: QK of T
        const int orow = ol & 31, oh = ol >> 5;
        const int ga = gperm(orow);
        const uint8_t* kq0 = kh + orow * RS + cbyte + 16 * (oh ^ (ga & 1)) + 32 * (ga >> 1);
        const uint8_t* kq1 = kh + orow * RS + cbyte + 16 * (oh ^ (ga & 1)) + 32 * ((ga >> 1) ^ 1);
        auto kread = [&](int s2) __attribute__((always_inline)) -> opvec {
            return *reinterpret_cast<const opvec*>(((s2 & 1) ? kq1 : kq0) + 64 * (s2 >> 1));
        };
        constexpr int QPF = 6;
        opvec kq[QPF];
#pragma unroll
        for (int s2 = 0; s2 < QPF; ++s2) kq[s2] = kread(s2);
        f32x16 st;
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = 0.0f;
        constexpr int DE = KW / NU;  // QK MFMAs per row copy of T+3
        static_assert(DE >= 1 && KW % NU == 0, "copies between the QK MFMAs");
#pragma unroll
        for (int s2 = 0; s2 < KW; ++s2) {
            const opvec av = kq[s2 % QPF];
            if (s2 + QPF < KW) kq[s2 % QPF] = kread(s2 + QPF);
            st = OP::mfma(av, qf[s2], st);
            if (s2 % DE == (DE > 1 ? 1 : 0) && s2 / DE < NU) dma_unit(s2 / DE);
        }
        // pinned order: the first reads, then each MFMA followed by the read
        // that runs ahead of it (else the prefetch collapses under pressure)
        __builtin_amdgcn_sched_group_barrier(0x100, QPF, 2);
#pragma unroll
        for (int s2 = 0; s2 < KW; ++s2) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
            if (s2 + QPF < KW) __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        exchange(st, true);
        __builtin_amdgcn_sched_barrier(0);
        // ---- B: logits relative to m_use (log2 units), P of the first keys
        if (__ballot(m_use == -INFINITY)) {  // first tile of the pass: m_use is its max
            float m0 = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) m0 = fmaxf(m0, st[r]);
            m0 = xor32_max(m0) * invq;
            m_use = (m_use == -INFINITY) ? m0 : m_use;
        }
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = __builtin_fmaf(st[r], invq, -m_use);
        uint32_t pk[8];
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; r += 2) {
            const float p0 = __builtin_amdgcn_exp2f(x[r]);
            const float p1 = __builtin_amdgcn_exp2f(x[r + 1]);
            psum += p0 + p1;
            pk[r >> 1] = OP::pack(p0, p1);
        }
        const opvec pa0 = __builtin_bit_cast(opvec, u32x4{pk[0], pk[1], pk[2], pk[3]});
        __builtin_amdgcn_sched_barrier(0);
        // ---- C: PV of T, k-step 0 over all column tiles, then k-step 1
        const int q = ol >> 4, i16 = ol & 15;
        const uint8_t* vrow[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int rr = 8 * hf + 4 * (q >> 1) + (i16 >> 2);
            vrow[hf] = kh + rr * RS + cbyte + 16 * ((2 * (q & 1) + ((i16 & 3) >> 1)) ^ gperm(rr)) + 8 * (i16 & 1);
        }
        auto vread = [&](int j) __attribute__((always_inline)) -> opvec {
            const int dt = j & (DW - 1), ks = j / DW;
            const int off = ks * 16 * RS + 64 * dt;
            const h4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4*)const_cast<uint8_t*>(vrow[0] + off));
            const h4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4*)const_cast<uint8_t*>(vrow[1] + off));
            const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
            return __builtin_bit_cast(opvec, u32x4{w0[0], w0[1], w1[0], w1[1]});
        };
        constexpr int VPF = 4, NJ = 2 * DW;
        static_assert(!PERM || NJ > 8, "the second keys' P, the max and the sums ride under the PV MFMAs");
        opvec vb[VPF];
#pragma unroll
        for (int j = 0; j < VPF; ++j) vb[j] = vread(j);
        opvec pa1;
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const opvec bv = vb[j % VPF];
            if (j + VPF < NJ) vb[j % VPF] = vread(j + VPF);
            if (j < DW) {
                acc[j] = OP::mfma(pa0, bv, acc[j]);
            } else {
                acc[j - DW] = OP::mfma(pa1, bv, acc[j - DW]);
            }
            // the second keys' P (needed from k-step 1 on), the max, the sums
            if (j >= 1 && j <= 4) {
                const int r = 8 + 2 * (j - 1);
                const float p0 = __builtin_amdgcn_exp2f(x[r]);
                const float p1 = __builtin_amdgcn_exp2f(x[r + 1]);
                psum += p0 + p1;
                pk[4 + (j - 1)] = OP::pack(p0, p1);
                if (j == 4) pa1 = __builtin_bit_cast(opvec, u32x4{pk[4], pk[5], pk[6], pk[7]});
            }
            if (j == 6) {
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[r]);
            }
            if (j == 8) {
                mx = xor32_max(mx);
                l_run += xor32_sum(psum);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * VPF, 0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (j + VPF < NJ) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        // the tile max only decides the flag and the second pass's m_use
        m_seen = fmaxf(m_seen, mx + m_use);
        if (__ballot(mx > 15.0f)) flagged = true;
        barrier_vm<NU>();  // all but T+3's loads have landed
    };
    // a step can take the fast form when its tile is full
    auto fast_tile = [&](int it) __attribute__((always_inline)) -> bool {
        return __builtin_amdgcn_readfirstlane(meta[it & (MS - 1)].mask) == 0xffffffffu;
    };

    for (int pass = 0; pass < 2; ++pass) {
        active = has_heads && (pass == 0 || flagged);
        if (pass == 1) {
            if (flagged) {
                m_use = m_seen;
                l_run = 0.0f;
                flagged = false;
            }
            meta_start();
            barrier_vm<0>();
            start_tiles();
        }
        if (active) {
#pragma unroll
            for (int dt = 0; dt < DW; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;
        }
        if (tile0 + 2 < tile1) barrier_vm<2 * NU>();
        else if (tile0 + 1 < tile1) barrier_vm<NU>();
        else barrier_vm<0>();
        if (tile0 < tile1) prep_tile(0, ring[0]);
        if (tile0 + 2 < tile1) barrier_vm<NU>();
        else barrier_vm<0>();
        {
            int it = 0;
            if constexpr (PERM && !RAW_F32) {
                for (; tile0 + it + 3 < tile1 && active && !flagged && fast_tile(it); ++it) step_fast(it);
            }
            for (; tile0 + it < tile1; ++it) step(it);
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
    // (lane indices re-derived here: nothing lane-dependent stays live across the loop)
    const int el = opaque_tid() & 63, erow = el & 31, eh = el >> 5;
    const int head = 32 * hbk + erow;
    const int dt0 = DW * chalf;  // first output dim tile of this wave
    if constexpr (FINAL) {
        // One split: the final output straight from the accumulator.  Per head,
        // in log2 units, Z = l + 2^(sink - m_use) and out = O / Z; the last r
        // channels are rotated back by -t (channel pairs sit in lanes 2i, 2i+1);
        // lse = ln 2 * (m_use + log2 Z).  No keys: out = 0, lse = the sink.
        if (el < 32) {
            const float sk = head < H ? sink_s[head] : -INFINITY;
            float zi = 0.0f, lse = sk;
            if (m_use != -INFINITY) {
                const float z = l_run + __builtin_amdgcn_exp2f(sk - m_use);
                zi = 1.0f / z;
                lse = m_use + __builtin_log2f(z);
            }
            il_s[wave][erow] = zi;
            if (head < H && a.lse && chalf == 0) a.lse[bq * H + head] = lse * 0.6931471805599453f;
        }
        f32x4 zi[4];  // 1/Z of this lane's accumulator rows 8 (r/4) + 4 eh + r%4
#pragma unroll
        for (int m = 0; m < 4; ++m) zi[m] = *reinterpret_cast<const f32x4*>(&il_s[wave][8 * m + 4 * eh]);
        // rope_dims <= 64, so only the last two column tiles hold rotated
        // channels; the rotation by -t reuses the query's table of +t
        float rsn[2], rcs[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int d = 32 * (DT - 2 + k) + erow;
            rsn[k] = 0.0f;
            rcs[k] = 1.0f;
            if (DT - 2 + k >= 0 && d >= rope_lo) {
                const float2 c = qcs[(d - rope_lo) >> 1];
                rcs[k] = c.x;
                rsn[k] = -c.y;
            }
        }
        // Rows r, r+1 of a column-pair of lanes (2i, 2i+1) become two 4-byte
        // bf16 pairs (8 bytes for f32): the even lane sends row r+1's value and
        // the odd lane row r's, so the even lane holds row r's channel pair and
        // the odd lane row r+1's.  bf16 rows are then staged in this wave's
        // (now idle) tile buffer and leave as whole rows, 16 bytes per lane;
        // the word index of rows 4..7 of each group of 8 is XORed with 32 so
        // that the four rows one write instruction touches use distinct banks.
        const bool odd = erow & 1;
        const bool f32o = a.out_f32 != 0;
        // the wave's 32 heads all exist (uniform): stores need no per-lane test
        const bool full = 32 * hbk + 32 <= H;
        uint8_t* ob = ring[wave];
        // (one unrolled pass per output type: a branch on the type inside the
        // unrolled loop costs a scalar branch and exec-mask set-up per store)
        // dt: this wave's output tile, dtg = dt0 + dt the row's
        auto out_rows = [&](auto&& put) __attribute__((always_inline)) {
#pragma unroll
        for (int dt = 0; dt < DW; ++dt) {
            const int dtg = dt0 + dt;
            const bool tile_rot = dtg >= DT - 2 && 32 * dtg + 32 > rope_lo;  // uniform
            const float sn = dtg == DT - 2 ? rsn[0] : (dtg == DT - 1 ? rsn[1] : 0.0f);
            const float cs = dtg == DT - 2 ? rcs[0] : (dtg == DT - 1 ? rcs[1] : 1.0f);
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                float v[2];
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    v[k] = acc[dt][r + k] * zi[(r + k) >> 2][(r + k) & 3];
                    if (tile_rot) {
                        const float o = lane_swap1(v[k]);  // the other channel of the pair
                        v[k] = odd ? o * sn + v[k] * cs : v[k] * cs - o * sn;
                    }
                }
                const float recv = lane_swap1(odd ? v[0] : v[1]);
                const float lo = odd ? recv : v[0], hi = odd ? v[1] : recv;
                const int row = 8 * (r >> 2) + 4 * eh + (r & 3) + (odd ? 1 : 0);
                put(dt, row, lo, hi);
            }
        }
        };
        if (f32o) {
            out_rows([&](int dt, int row, float lo, float hi) __attribute__((always_inline)) {
                const int hr = 32 * hbk + row;
                if (hr < H)
                    *reinterpret_cast<float2*>(reinterpret_cast<float*>(a.out) + (bq * H + hr) * (int64_t)D +
                                               32 * (dt0 + dt) + (erow & ~1)) = make_float2(lo, hi);
            });
        } else {
            // the wave's part of a row (all of it, or one channel half) is
            // staged as DW * 16 words
            out_rows([&](int dt, int row, float lo, float hi) __attribute__((always_inline)) {
                const int word = (16 * dt + (erow >> 1)) ^ (((row >> 2) & 1) << 5);
                *reinterpret_cast<uint32_t*>(ob + row * RS + 4 * word) = pack_bf16x2(lo, hi);
            });
            constexpr int LPRO = DW * 32 / 8;  // lanes per bf16 output row part (16 bytes each)
            constexpr int RPI = 64 / LPRO;     // rows per instruction
#pragma unroll
            for (int h0 = 0; h0 < 32; h0 += RPI) {
                const int h = h0 + el / LPRO, c = el % LPRO;
                const int hr = 32 * hbk + h;
                const u32x4 w = *reinterpret_cast<const u32x4*>(ob + h * RS + 4 * ((4 * c) ^ (((h >> 2) & 1) << 5)));
                if (full || hr < H)
                    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + (bq * H + hr) * (int64_t)D +
                                              32 * dt0 + 8 * c) = w;
            }
        }
        return;
    }
    // Several splits: (max, sum) of this split and its output normalised by its
    // own sum, O/l (a convex combination of normalised rows, so fp16 holds it),
    // with the heads of an even/odd pair packed in one word.  The combine
    // kernel folds in the sink, merges the splits, rotates back and stores.
    const int S = a.n_splits;
    const int64_t base = (bq * S + split) * (int64_t)H;
    if (el < 32) {
        if (head < H && chalf == 0) {
            a.part_ml[(base + head) * 2] = m_use;
            a.part_ml[(base + head) * 2 + 1] = l_run;
        }
        il_s[wave][erow] = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    }
    f32x4 il[4];  // 1/l of this lane's accumulator rows 8 (r/4) + 4 eh + r%4
#pragma unroll
    for (int m = 0; m < 4; ++m) il[m] = *reinterpret_cast<const f32x4*>(&il_s[wave][8 * m + 4 * eh]);
    const int64_t pbase = (bq * S + split) * (int64_t)((H + 1) >> 1);
    // (a wave whose 32 heads all exist stores without a per-lane test)
    auto put_partials = [&](bool check) __attribute__((always_inline)) {
#pragma unroll
        for (int dt = 0; dt < DW; ++dt)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int hr = 32 * hbk + 8 * (r >> 2) + 4 * eh + (r & 3);  // even
                if (!check || hr < H)
                    a.part_o[(pbase + (hr >> 1)) * D + 32 * (dt0 + dt) + erow] =
                        pack_f16x2(acc[dt][r] * il[r >> 2][r & 3], acc[dt][r + 1] * il[r >> 2][(r & 3) + 1]);
            }
    };
    if (32 * hbk + 32 <= H) put_partials(false);
    else put_partials(true);
}

// Merge split partials: one workgroup per (query, head pair), one thread per
// channel pair (so the inverse rotation of a pair stays in one thread).  One
// pass over the splits with a running maximum (log2 units): the loads of
// eight splits are issued before any of their arithmetic.
template <int D>
__global__ __launch_bounds__(256) void mqa_combine_kernel(const AttnArgs a) {
    constexpr int SB = 8;  // splits per batch of loads
    const int H = a.H, Hp = (H + 1) >> 1;
    const int64_t wg = xcd_order(blockIdx.x, gridDim.x);
    const int64_t bq = wg / Hp;
    const int hp = (int)(wg % Hp);
    const int S = a.n_splits;
    const int pr = threadIdx.x;  // pair index
    if (2 * pr >= D) return;
    const int nh = (2 * hp + 1 < H) ? 2 : 1;
    const float LOG2E = 1.4426950408889634f;
    float M[2], Z[2], o[2][2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int h = 2 * hp + (e < nh ? e : 0);
        M[e] = a.sinks[h] * LOG2E;
        Z[e] = M[e] == -INFINITY ? 0.0f : 1.0f;
        o[e][0] = o[e][1] = 0.0f;
    }
    const uint2* po = reinterpret_cast<const uint2*>(a.part_o) + (bq * S * Hp + hp) * (int64_t)(D / 2) + pr;
    const float2* pml = reinterpret_cast<const float2*>(a.part_ml) + bq * S * H + 2 * hp;
    for (int s0 = 0; s0 < S; s0 += SB) {
        uint2 wv[SB];
        float2 ml[SB][2];
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int s = s0 + j < S ? s0 + j : S - 1;  // past the end: repeat the last, unused
            wv[j] = po[(int64_t)s * Hp * (D / 2)];
            ml[j][0] = pml[(int64_t)s * H];
            ml[j][1] = pml[(int64_t)s * H + (nh > 1 ? 1 : 0)];
        }
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            if (s0 + j >= S) break;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                if (e >= nh) continue;
                const float ms = ml[j][e].x;
                if (ms == -INFINITY) continue;
                const float mn = fmaxf(M[e], ms);
                const float keep = M[e] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M[e] - mn);
                const float wl = __builtin_amdgcn_exp2f(ms - mn) * ml[j][e].y;
                const float v0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(e ? wv[j].x >> 16 : wv[j].x & 0xffffu));
                const float v1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(e ? wv[j].y >> 16 : wv[j].y & 0xffffu));
                Z[e] = __builtin_fmaf(Z[e], keep, wl);
                o[e][0] = __builtin_fmaf(wl, v0, o[e][0] * keep);
                o[e][1] = __builtin_fmaf(wl, v1, o[e][1] * keep);
                M[e] = mn;
            }
        }
    }
    const int rope_lo = D - a.rope_dims;
    float sn = 0.0f, cs = 1.0f;
    if (2 * pr >= rope_lo) {
        int32_t t = a.q_pos[bq];
        t = t < 0 ? 0 : t;
        sincos_turns(-(double)t * rope_turns(a.rope_ratio, (2 * pr - rope_lo) >> 1), &sn, &cs);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        if (e >= nh) continue;
        const int h = 2 * hp + e;
        float o0 = Z[e] > 0.0f ? o[e][0] / Z[e] : 0.0f, o1 = Z[e] > 0.0f ? o[e][1] / Z[e] : 0.0f;
        if (2 * pr >= rope_lo) {
            const float x0 = o0, x1 = o1;
            o0 = x0 * cs - x1 * sn;
            o1 = x0 * sn + x1 * cs;
        }
        const int64_t off = (bq * H + h) * (int64_t)D + 2 * pr;
        if (a.out_f32) {
            *reinterpret_cast<float2*>(reinterpret_cast<float*>(a.out) + off) = make_float2(o0, o1);
        } else {
            reinterpret_cast<uint32_t*>(a.out)[off >> 1] = pack_bf16x2(o0, o1);
        }
        if (pr == 0 && a.lse)
            a.lse[bq * H + h] = (M[e] == -INFINITY) ? -INFINITY : (M[e] + __builtin_log2f(Z[e])) * 0.6931471805599453f;
    }
}

template <int D, bool SPARSE, typename TIn, bool CS>
static int launch_one(const AttnArgs& a, int64_t BQ, hipStream_t stream) {
    dim3 grid((unsigned)a.n_splits, (unsigned)BQ);
    prof_mark("mqa_fwd_kernel", false, stream);
    if (a.n_splits == 1)
        hipLaunchKernelGGL((mqa_fwd_kernel<D, SPARSE, TIn, true, CS>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((mqa_fwd_kernel<D, SPARSE, TIn, false, CS>), grid, dim3(256), 0, stream, a);
    prof_mark("mqa_fwd_kernel", true, stream);
    if (hipGetLastError() != hipSuccess) return -4;
    if (a.n_splits == 1) return 0;  // the forward kernel wrote the output itself
    prof_mark("mqa_combine_kernel", false, stream);
    hipLaunchKernelGGL((mqa_combine_kernel<D>), dim3((unsigned)(BQ * ((a.H + 1) / 2))), dim3(D / 2 < 64 ? 64 : D / 2),
                       0, stream, a);
    prof_mark("mqa_combine_kernel", true, stream);
    if (hipGetLastError() != hipSuccess) return -4;
    return 0;
}

template <int D>
static int launch_d(const AttnArgs& a, int64_t BQ, bool act_f32, hipStream_t stream) {
    const bool sparse = a.idx != nullptr;
    if constexpr (D <= 128) {
        if (act_f32)
            return sparse ? launch_one<D, true, float, false>(a, BQ, stream)
                          : launch_one<D, false, float, false>(a, BQ, stream);
    } else {
        if (act_f32) return -2;  // f32 activations: head dims up to 128
        // up to 64 heads: the channel-split geometry keeps all four waves busy
        if (a.H <= 64)
            return sparse ? launch_one<D, true, bf16_t, true>(a, BQ, stream)
                          : launch_one<D, false, bf16_t, true>(a, BQ, stream);
    }
    return sparse ? launch_one<D, true, bf16_t, false>(a, BQ, stream) : launch_one<D, false, bf16_t, false>(a, BQ, stream);
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
