// cakv_internal.hpp -- host-side launcher interfaces between the C ABI layer
// (api.cpp) and the kernel translation units.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cakv {

constexpr int kMaxRopePairs = 32;  // rope_dims <= 64
constexpr int kTopkCap = 4096;     // largest k
constexpr int kCandCap = 8192;     // entries of the threshold bin listed per query on the fast path
constexpr int kHistBins = 2048;    // 11-bit histogram levels over the score key
constexpr int kHistStride = 2 * kHistBins + 64;  // words per query: level 1, level 2, counter

// Everything one attention launch needs; passed by value as the kernel
// argument block.
struct AttnArgs {
    const void* q;
    const void* kv_c;
    const int32_t* idx;  // NULL for the dense path
    const void* kv_raw;
    const int32_t* raw_pos0;
    const int32_t* q_pos;
    const float* sinks;
    const float* gamma_q;
    void* out;
    float* lse;
    uint32_t* part_o;  // [BQ][S][(H+1)/2][D] split outputs O/l, fp16, heads (2p, 2p+1) in one word
    float* part_ml;  // [BQ][S][H][2]   split partial (max, sum), max in log2 units
    int64_t Q;
    int64_t N;
    int64_t R;
    int32_t H;
    int32_t K;
    int32_t m;
    int32_t n_win;
    int32_t rope_dims;
    float scale_log2;  // softmax scale * log2(e)
    float rms_eps;
    int32_t n_splits;
    int32_t out_f32;   // 1: float32 output, 0: bf16
    int32_t raw_ring;  // 1: kv_raw row p mod R holds position p (raw_pos0 unused)
    double rope_ratio; // rope_base^(-2/rope_dims), so theta_i = rope_ratio^i
};

// rope_base^(-2/rope_dims) in fp64 (host side; 1 when nothing rotates)
inline double rope_ratio_of(float rope_base, int rope_dims) {
    return rope_dims > 0 ? pow((double)rope_base, -2.0 / (double)rope_dims) : 1.0;
}

// theta_i / (2 pi) in fp64: turns of rotary pair i per unit of position,
// theta_i = ratio^i by repeated squaring (relative error ~1e-15, far below
// what the fp32 sine and cosine resolve)
__device__ __forceinline__ double rope_turns(double ratio, int i) {
    double r = 1.0, b = ratio;
    for (int e = i; e > 0; e >>= 1) {
        if (e & 1) r *= b;
        b *= b;
    }
    return r * 0.15915494309189533577;
}

// entry j covers tokens [max(0, (j+1)m - span), (j+1)m); gate [B,T] or, with
// gate_per_channel, [B,T,D]
int launch_kv_compress(const void* x, int x_dtype, const float* gate, bool gate_per_channel, int64_t B,
                       int64_t T, int64_t D, int32_t m, int32_t span, void* out, int out_dtype,
                       float* out_scale, hipStream_t stream);

// dtype 0: float32, 1: bf16; entries j0 .. j0+n-1 of each of the B sequences
int launch_kv_prepare(const void* in, void* out, int dtype, int64_t B, int64_t N, int64_t D, int64_t j0,
                      int64_t n, const float* gamma, int32_t m, int32_t rope_dims, double rope_ratio,
                      int32_t pos_off, float eps, hipStream_t stream);

// One streaming append (cakv_kv_append): a new token per sequence enters one
// compressor's rings and, when it completes a block, its cache.
struct AppendArgs {
    const void* x_tok;      // [B][D] act
    const float* gate_tok;  // [B] or [B][D]
    const int32_t* pos;     // [B]
    void* raw_ring;         // [B][Rr][D] act
    float* gate_ring;       // [B][Rr] or [B][Rr][D]
    void* win_ring;         // [B][Rw][D] act, prepared rows, or NULL
    void* cache;            // [B][N][D] act (prepared when prep) or fp8 codes
    float* cache_scale;     // [B][N] fp8 only
    const float* gamma_kv;  // [D] or NULL
    int64_t Rr;
    int64_t Rw;
    int64_t N;
    int32_t D;
    int32_t m;
    int32_t span;
    int32_t prep;           // 1: cache entries are prepared (RMSNorm + RoPE)
    int32_t rope_dims;
    int32_t pos_off;        // entry j sits at position j*m + pos_off
    float eps;
    double rope_ratio;
};

// act_dtype / cache_dtype: 0 f32, 1 bf16, 2 fp8 (cache only)
int launch_kv_append(const AppendArgs& a, int64_t B, int act_dtype, int cache_dtype, bool gate_per_channel,
                     hipStream_t stream);

// up to kAppendBatchMax appends of the same B tokens in one launch; kind[y] =
// 4 * (activations bf16) + 2 * (cache fp8) + (per-channel gates)
constexpr int kAppendBatchMax = 4;
struct AppendBatch {
    AppendArgs a[kAppendBatchMax];
    int32_t kind[kAppendBatchMax];
};
int launch_kv_append_batch(const AppendBatch& ab, int32_t n, int64_t B, hipStream_t stream);

// sparse (idx != NULL) or dense MQA forward; act_f32: inputs are float32
int launch_mqa_fwd(const AttnArgs& a, int64_t BQ, int D, bool act_f32, hipStream_t stream);

// Profiling aid (cakv_profile_kernel_events): record the calling thread's
// pending start (after = false) or end event around a launch of `kernel`.
void prof_mark(const char* kernel, bool after, hipStream_t stream);

struct IndexerArgs {
    const void* q_idx;
    const float* w;
    const void* k_idx;
    const float* k_scale;
    const int32_t* q_pos;
    int32_t* idx;
    const void* kpack;   // fp8 keys repacked for the score kernel when Q > 1 (see indexer.hip), else NULL
    uint32_t* keys;      // [BQ][N] order-preserving score keys
    uint32_t* hist;      // [BQ][kHistStride] key histograms (top 11 bits; next 11 bits) + counters
    uint32_t* cand_a;    // [BQ][kTopkCap] entries above the threshold bin
    uint64_t* cand_b;    // [BQ][kCandCap] rank values (~key << 32 | j) of the entries in the threshold bin
    int64_t Q;
    int64_t N;
    int32_t HI;
    int32_t dI;
    int32_t m;
    int32_t k;
    int32_t chunk;       // entries per score workgroup
    int32_t n_chunks;
};

// Attention backward: the forward's arguments plus the gradients and the
// workspace arrays (laid out by launch_mqa_bwd).
struct BwdArgs {
    AttnArgs f;
    const void* out;    // forward output [BQ][H][D], bf16 or f32 (out_f32)
    const float* lse;   // [BQ][H]
    const float* dout;  // [BQ][H][D]
    float* dq;          // [BQ][H][D], written
    float* dkv_c;       // [B][N][D], accumulated
    float* dkv_raw;     // [B][R][D], accumulated
    float* dsinks;      // [H], accumulated, or NULL
    float* dgamma_q;    // [D], accumulated, or NULL
    uint16_t* qh;       // [BQ][HP][D] bf16 q_hat
    uint16_t* doh;      // [BQ][HP][D] bf16 do = RoPE_t(dout)
    uint16_t* qt;       // [BQ][D][HP] bf16 q_hat transposed
    uint16_t* dot;      // [BQ][D][HP] bf16 do transposed
    float* delta;       // [BQ][H] do . o
    uint16_t* pt;       // [BQ][S][HP] bf16 P (key-major)
    uint16_t* dlt;      // [BQ][S][HP] bf16 tau * dl (key-major)
    uint16_t* dl;       // [BQ][HP][S] bf16 dl (head-major)
    int32_t out_f32;
    int32_t unique_rows;  // 1: one query per sequence (no row is touched by two workgroups)
    int32_t HP;         // heads rounded up to 32
    int32_t S;          // key slots per query, rounded up to 32
    float tau;          // softmax scale
};
size_t mqa_bwd_workspace_bytes(int64_t BQ, int32_t H, int64_t max_slots, int n_splits);
int launch_mqa_bwd(BwdArgs& w, int64_t BQ, int64_t max_slots, void* ws, hipStream_t stream);

// dtype 0: float32, 1: bf16; dy, dx: [B][N][D] float32, rows j0 .. j0+n-1
int launch_kv_prepare_bwd(const void* in, const float* dy, float* dx, float* dgamma, int dtype, int64_t B, int64_t N,
                          int64_t D, int64_t j0, int64_t n, const float* gamma, int32_t m, int32_t rope_dims,
                          double rope_ratio, int32_t pos_off, float eps, hipStream_t stream);

size_t kv_compress_bwd_workspace_bytes(int64_t B, int64_t T, int64_t D, int32_t m);
int launch_kv_compress_bwd(const void* x, int x_dtype, const float* gate, bool pc, int64_t B, int64_t T, int64_t D,
                           int32_t m, int32_t span, const float* dc, float* dx, float* dgate, void* ws,
                           hipStream_t stream);

struct IndexerBwdArgs {
    const void* q_idx;    // [BQ][HI][dI] f32 or bf16
    const float* w;       // [BQ][HI]
    const void* k_idx;    // [B][N][dI] f32 or fp8 codes
    const float* k_scale; // [B][N] (fp8)
    const int32_t* q_pos; // [BQ]
    const int32_t* idx;   // [BQ][K]
    const float* dS;      // [BQ][K]
    float* dq;            // [BQ][HI][dI], written
    float* dw;            // [BQ][HI], written
    float* dk;            // [B][N][dI], accumulated
    int64_t Q;
    int64_t N;
    int32_t HI;
    int32_t dI;
    int32_t m;
    int32_t K;
};
int launch_indexer_bwd(const IndexerBwdArgs& a, int64_t BQ, bool q_f32, bool fp8, hipStream_t stream);

size_t indexer_workspace_bytes(int64_t B, int64_t Q, int64_t N, int32_t k);
int launch_indexer_topk(IndexerArgs& a, int64_t BQ, bool fp8_mode, void* ws, hipStream_t stream);

}  // namespace cakv
