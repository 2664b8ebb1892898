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

int launch_kv_compress(const void* x, int x_dtype, const float* gate, int64_t B, int64_t T,
                       int64_t D, int32_t m, void* out, int out_dtype, float* out_scale,
                       hipStream_t stream);

// dtype 0: float32, 1: bf16; entries j0 .. j0+n-1 of each of the B sequences
int launch_kv_prepare(const void* in, void* out, int dtype, int64_t B, int64_t N, int64_t D, int64_t j0,
                      int64_t n, const float* gamma, int32_t m, int32_t rope_dims, double rope_ratio,
                      int32_t pos_off, float eps, hipStream_t stream);

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

size_t indexer_workspace_bytes(int64_t BQ, int64_t N, int32_t k);
int launch_indexer_topk(IndexerArgs& a, int64_t BQ, bool fp8_mode, void* ws, hipStream_t stream);

}  // namespace cakv
