// api.hip -- the C ABI of the compressed-attention library (include/cakv.h):
// argument validation, workspace sizing, launch geometry.  Every check runs
// before anything is enqueued; on error nothing is launched.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>
#include <vector>

#include "../../include/cakv.h"
#include "cakv_internal.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return CAKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, code, ...) \
    do {                         \
        if (!(cond)) return fail(code, __VA_ARGS__); \
    } while (0)

#define REQUIRE_PTR(p, name)                                                 \
    do {                                                                     \
        if (!(p)) return fail(CAKV_EINVAL, "%s must not be NULL", name);    \
        if (!aligned16(p)) return fail(CAKV_EINVAL, "%s must be 16-byte aligned", name); \
    } while (0)

int rc_from(int r) {
    if (r == 0) return ok();
    if (r == -2) return fail(CAKV_EUNSUPPORTED, "unsupported launch configuration");
    return fail(CAKV_ELAUNCH, "kernel launch failed: %s", hipGetErrorString(hipGetLastError()));
}

constexpr int kTK = 32;  // attention key slots per tile

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// splits over key tiles for one attention launch: enough workgroups to cover
// the 256 compute units, but at least four tiles per split so the per-query
// prologue stays amortised
int attn_splits(int64_t BQ, int64_t max_slots) {
    if (BQ <= 0) return 1;
    const int64_t tiles = ceil_div(max_slots, kTK);
    int64_t s = ceil_div(256, BQ);
    const int64_t cap = tiles / 4 > 1 ? tiles / 4 : 1;
    if (s > cap) s = cap;
    if (s < 1) s = 1;
    if (s > 64) s = 64;
    return (int)s;
}

size_t attn_workspace(int64_t BQ, int32_t H, int32_t D, int64_t max_slots) {
    const int S = attn_splits(BQ, max_slots);
    if (S == 1) return 0;  // one split: the forward kernel writes the output itself
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return al((size_t)BQ * S * ((H + 1) / 2) * D * 4) + al((size_t)BQ * S * H * 2 * 4);
}

int check_attn_common(const cakv_attn_params* p, const void* q, const void* kv_c, const void* kv_raw,
                      const int32_t* raw_pos0, const int32_t* q_pos, const float* sinks, int act_dtype,
                      int64_t B, int64_t Q, int32_t H, int32_t D, int64_t N, int64_t R, void* out,
                      int out_dtype, float* lse) {
    REQUIRE(p, CAKV_EINVAL, "params must not be NULL");
    REQUIRE(B >= 0 && Q >= 0 && N >= 0 && R >= 0, CAKV_EINVAL, "negative size (B=%lld Q=%lld N=%lld R=%lld)",
            (long long)B, (long long)Q, (long long)N, (long long)R);
    REQUIRE(H >= 1 && H <= 128, CAKV_EUNSUPPORTED, "H=%d: 1 <= H <= 128 supported", H);
    REQUIRE(D == 128 || D == 512, CAKV_EUNSUPPORTED, "D=%d: head dims 128 and 512 supported", D);
    REQUIRE(act_dtype == CAKV_BF16 || act_dtype == CAKV_F32, CAKV_EINVAL, "act_dtype must be BF16 or F32");
    REQUIRE(act_dtype == CAKV_BF16 || D <= 128, CAKV_EUNSUPPORTED, "F32 activations support D <= 128 (D=%d)", D);
    REQUIRE(out_dtype == CAKV_BF16 || out_dtype == CAKV_F32, CAKV_EINVAL, "out_dtype must be BF16 or F32");
    REQUIRE(p->m >= 1 && p->m <= 4096, CAKV_EUNSUPPORTED, "m=%d out of 1..4096", p->m);
    REQUIRE(p->n_win >= 0 && p->n_win <= 4096, CAKV_EUNSUPPORTED, "n_win=%d out of 0..4096", p->n_win);
    REQUIRE(p->rope_dims >= 0 && p->rope_dims <= 2 * cakv::kMaxRopePairs && (p->rope_dims & 1) == 0 &&
                p->rope_dims <= D,
            CAKV_EUNSUPPORTED, "rope_dims=%d: even, <= %d and <= D", p->rope_dims, 2 * cakv::kMaxRopePairs);
    REQUIRE(p->rope_base > 0.0f && isfinite(p->rope_base), CAKV_EINVAL, "rope_base must be positive");
    REQUIRE(p->softmax_scale >= 0.0f && isfinite(p->softmax_scale), CAKV_EINVAL, "softmax_scale must be >= 0");
    REQUIRE(p->rms_eps >= 0.0f && isfinite(p->rms_eps), CAKV_EINVAL, "rms_eps must be >= 0");
    if (B * Q == 0) return CAKV_OK;
    REQUIRE_PTR(q, "q");
    REQUIRE_PTR(raw_pos0, "raw_pos0");
    REQUIRE_PTR(q_pos, "q_pos");
    REQUIRE_PTR(sinks, "sinks");
    REQUIRE_PTR(out, "out");
    if (N > 0) REQUIRE_PTR(kv_c, "kv_c");
    if (R > 0) REQUIRE_PTR(kv_raw, "kv_raw");
    if (lse) REQUIRE(aligned16(lse), CAKV_EINVAL, "lse must be 16-byte aligned");
    if (p->gamma_q) REQUIRE(aligned16(p->gamma_q), CAKV_EINVAL, "gamma_q must be 16-byte aligned");
    REQUIRE(B * Q <= 0x7fffffffLL, CAKV_EUNSUPPORTED, "B*Q too large");
    return CAKV_OK;
}

void fill_attn(cakv::AttnArgs& a, const cakv_attn_params* p, const void* q, const void* kv_c,
               const int32_t* idx, const void* kv_raw, const int32_t* raw_pos0, const int32_t* q_pos,
               const float* sinks, int64_t Q, int32_t H, int32_t D, int64_t N, int32_t K, int64_t R,
               void* out, int out_dtype, float* lse) {
    a.q = q;
    a.kv_c = kv_c;
    a.idx = idx;
    a.kv_raw = kv_raw;
    a.raw_pos0 = raw_pos0;
    a.q_pos = q_pos;
    a.sinks = sinks;
    a.gamma_q = p->gamma_q;
    a.out = out;
    a.lse = lse;
    a.part_o = nullptr;
    a.part_ml = nullptr;
    a.Q = Q;
    a.N = N;
    a.R = R;
    a.H = H;
    a.K = K;
    a.m = p->m;
    a.n_win = p->n_win;
    a.rope_dims = p->rope_dims;
    const double tau = p->softmax_scale > 0.0f ? (double)p->softmax_scale : 1.0 / sqrt((double)D);
    a.scale_log2 = (float)(tau * 1.4426950408889634);
    a.rms_eps = p->rms_eps;
    a.out_f32 = out_dtype == CAKV_F32;
    a.rope_ratio = cakv::rope_ratio_of(p->rope_base, p->rope_dims);
}

int run_attn(cakv::AttnArgs& a, int64_t BQ, int32_t H, int32_t D, int64_t max_slots, bool act_f32,
             void* ws, size_t ws_bytes, void* stream) {
    const int S = attn_splits(BQ, max_slots);
    const size_t need = attn_workspace(BQ, H, D, max_slots);
    REQUIRE(ws_bytes >= need, CAKV_EWORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
    if (need > 0) {
        REQUIRE(ws && (reinterpret_cast<uintptr_t>(ws) & 255u) == 0, CAKV_EWORKSPACE,
                "workspace must be non-NULL and 256-byte aligned");
        a.part_o = reinterpret_cast<uint32_t*>(ws);
        a.part_ml = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) +
                                             (((size_t)BQ * S * ((H + 1) / 2) * D * 4 + 255) & ~(size_t)255));
    }
    a.n_splits = S;
    return rc_from(cakv::launch_mqa_fwd(a, BQ, D, act_f32, reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

namespace cakv {

// Pending kernel-event pairs of the calling thread (cakv_profile_kernel_events).
struct ProfEvents {
    std::string kernel;
    std::vector<hipEvent_t> starts, ends;
    size_t next = 0;
};
thread_local ProfEvents g_prof;

void prof_mark(const char* kernel, bool after, hipStream_t stream) {
    if (g_prof.next >= g_prof.starts.size() || g_prof.kernel != kernel) return;
    (void)hipEventRecord(after ? g_prof.ends[g_prof.next] : g_prof.starts[g_prof.next], stream);
    if (after) ++g_prof.next;
}

}  // namespace cakv

extern "C" {

int cakv_version(void) { return 100; }

int cakv_profile_kernel_events(const char* kernel, void* const* starts, void* const* ends, int n) {
    REQUIRE(n >= 0, CAKV_EINVAL, "n=%d must be >= 0", n);
    cakv::g_prof = cakv::ProfEvents{};
    if (n == 0 || kernel == nullptr) return ok();
    REQUIRE(starts && ends, CAKV_EINVAL, "starts and ends must not be NULL when n > 0");
    for (int i = 0; i < n; ++i) REQUIRE(starts[i] && ends[i], CAKV_EINVAL, "event %d is NULL", i);
    cakv::g_prof.kernel = kernel;
    for (int i = 0; i < n; ++i) {
        cakv::g_prof.starts.push_back(reinterpret_cast<hipEvent_t>(starts[i]));
        cakv::g_prof.ends.push_back(reinterpret_cast<hipEvent_t>(ends[i]));
    }
    return ok();
}

const char* cakv_last_error(void) { return g_err.c_str(); }

int cakv_kv_compress(const void* x, int x_dtype, const float* gate, int64_t B, int64_t T, int64_t D,
                     int32_t m, void* out, int out_dtype, float* out_scale, void* stream) {
    REQUIRE(B >= 0 && T >= 0, CAKV_EINVAL, "negative size (B=%lld T=%lld)", (long long)B, (long long)T);
    REQUIRE(m >= 1 && m <= 4096, CAKV_EUNSUPPORTED, "m=%d out of 1..4096", m);
    REQUIRE(D >= 4 && D <= 4096 && D % 4 == 0, CAKV_EUNSUPPORTED, "D=%lld: 4..4096, a multiple of 4", (long long)D);
    REQUIRE(x_dtype == CAKV_F32 || x_dtype == CAKV_BF16, CAKV_EINVAL, "x_dtype must be F32 or BF16");
    REQUIRE(out_dtype == CAKV_F32 || out_dtype == CAKV_BF16 || out_dtype == CAKV_FP8_E4M3, CAKV_EINVAL,
            "out_dtype must be F32, BF16 or FP8_E4M3");
    REQUIRE((out_dtype == CAKV_FP8_E4M3) == (out_scale != nullptr), CAKV_EINVAL,
            "out_scale is required for FP8_E4M3 output and must be NULL otherwise");
    if (B * (T / m) == 0) return ok();
    REQUIRE_PTR(x, "x");
    REQUIRE_PTR(gate, "gate");
    REQUIRE_PTR(out, "out");
    if (out_scale) REQUIRE(aligned16(out_scale), CAKV_EINVAL, "out_scale must be 16-byte aligned");
    return rc_from(cakv::launch_kv_compress(x, x_dtype, gate, B, T, D, m, out, out_dtype, out_scale,
                                            reinterpret_cast<hipStream_t>(stream)));
}

int cakv_kv_prepare(const void* kv_in, void* kv_out, int act_dtype, int64_t B, int64_t N, int64_t D,
                    int64_t j0, int64_t n, const float* gamma_kv, int32_t m, int32_t rope_dims, float rope_base,
                    int32_t entry_pos_offset, float rms_eps, void* stream) {
    REQUIRE(B >= 0 && N >= 0 && j0 >= 0 && n >= 0 && j0 + n <= N, CAKV_EINVAL,
            "entries [%lld, %lld) outside 0..N=%lld (B=%lld)", (long long)j0, (long long)(j0 + n), (long long)N,
            (long long)B);
    REQUIRE(act_dtype == CAKV_F32 || act_dtype == CAKV_BF16, CAKV_EINVAL, "act_dtype must be F32 or BF16");
    REQUIRE(D >= 8 && D <= 4096 && D % 8 == 0, CAKV_EUNSUPPORTED, "D=%lld: 8..4096, a multiple of 8", (long long)D);
    REQUIRE(m >= 1, CAKV_EINVAL, "m=%d must be >= 1", m);
    REQUIRE(rope_dims >= 0 && (rope_dims & 1) == 0 && rope_dims <= D, CAKV_EINVAL, "rope_dims=%d: even, 0..D",
            rope_dims);
    REQUIRE(rope_base > 0.0f && isfinite(rope_base), CAKV_EINVAL, "rope_base must be positive");
    REQUIRE(rms_eps >= 0.0f && isfinite(rms_eps), CAKV_EINVAL, "rms_eps must be >= 0");
    REQUIRE((N - 1) * (int64_t)m + entry_pos_offset <= 0x7fffffffLL && entry_pos_offset >= -0x7fffffffLL,
            CAKV_EINVAL, "entry positions must fit in int32");
    if (B * n == 0) return ok();
    REQUIRE_PTR(kv_in, "kv_in");
    REQUIRE_PTR(kv_out, "kv_out");
    if (gamma_kv) REQUIRE(aligned16(gamma_kv), CAKV_EINVAL, "gamma_kv must be 16-byte aligned");
    return rc_from(cakv::launch_kv_prepare(kv_in, kv_out, act_dtype == CAKV_F32 ? 0 : 1, B, N, D, j0, n, gamma_kv,
                                           m, rope_dims, cakv::rope_ratio_of(rope_base, rope_dims), entry_pos_offset, rms_eps,
                                           reinterpret_cast<hipStream_t>(stream)));
}

size_t cakv_indexer_topk_workspace(int64_t B, int64_t Q, int64_t N, int32_t k) {
    if (B < 0 || Q < 0 || N < 0 || k < 1) return 0;
    return cakv::indexer_workspace_bytes(B * Q, N, k);
}

int cakv_indexer_topk(const void* q_idx, int q_dtype, const float* w, const void* k_idx, int k_dtype,
                      const float* k_scale, const int32_t* q_pos, int64_t B, int64_t Q, int64_t N,
                      int32_t HI, int32_t dI, int32_t m, int32_t k, int32_t* idx, void* workspace,
                      size_t workspace_bytes, void* stream) {
    REQUIRE(B >= 0 && Q >= 0 && N >= 0, CAKV_EINVAL, "negative size");
    REQUIRE(m >= 1, CAKV_EINVAL, "m=%d must be >= 1", m);
    REQUIRE(k >= 1 && k <= cakv::kTopkCap, CAKV_EUNSUPPORTED, "k=%d out of 1..%d", k, cakv::kTopkCap);
    REQUIRE(N <= 0x7fffffffLL, CAKV_EUNSUPPORTED, "N too large");
    const bool f32 = q_dtype == CAKV_F32 && k_dtype == CAKV_F32;
    const bool fp8 = q_dtype == CAKV_BF16 && k_dtype == CAKV_FP8_E4M3;
    REQUIRE(f32 || fp8, CAKV_EUNSUPPORTED, "dtypes: (F32 q, F32 k) or (BF16 q, FP8_E4M3 k)");
    if (f32) {
        REQUIRE(HI >= 1 && HI <= 64 && dI >= 4 && dI % 4 == 0 && HI * dI <= 8192, CAKV_EUNSUPPORTED,
                "fp32 mode: HI <= 64, dI a multiple of 4, HI*dI <= 8192 (HI=%d dI=%d)", HI, dI);
        REQUIRE(k_scale == nullptr, CAKV_EINVAL, "k_scale must be NULL for F32 keys");
    } else {
        REQUIRE((HI == 32 || HI == 64) && (dI == 64 || dI == 128), CAKV_EUNSUPPORTED,
                "fp8 mode: HI in {32,64}, dI in {64,128} (HI=%d dI=%d)", HI, dI);
    }
    const int64_t BQ = B * Q;
    if (BQ == 0) return ok();
    REQUIRE(BQ <= 0x7fffffffLL, CAKV_EUNSUPPORTED, "B*Q too large");
    REQUIRE_PTR(q_idx, "q_idx");
    REQUIRE_PTR(w, "w");
    REQUIRE_PTR(q_pos, "q_pos");
    REQUIRE_PTR(idx, "idx");
    if (N > 0) {
        REQUIRE_PTR(k_idx, "k_idx");
        if (fp8) REQUIRE_PTR(k_scale, "k_scale");
    }
    const size_t need = cakv::indexer_workspace_bytes(BQ, N, k);
    REQUIRE(workspace_bytes >= need, CAKV_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    REQUIRE(workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, CAKV_EWORKSPACE,
            "workspace must be non-NULL and 256-byte aligned");
    cakv::IndexerArgs a{};
    a.q_idx = q_idx;
    a.w = w;
    a.k_idx = k_idx;
    a.k_scale = k_scale;
    a.q_pos = q_pos;
    a.idx = idx;
    a.Q = Q;
    a.N = N;
    a.HI = HI;
    a.dI = dI;
    a.m = m;
    a.k = k;
    // score chunks: ~512 workgroups in total (two resident per CU), 128-entry granules
    const int64_t units = N > 0 ? ceil_div(N, 128) : 1;
    int64_t per_q = ceil_div(512, BQ);
    if (per_q > units) per_q = units;
    if (per_q < 1) per_q = 1;
    a.chunk = (int32_t)(ceil_div(units, per_q) * 128);
    a.n_chunks = (int32_t)ceil_div(N > 0 ? N : 1, a.chunk);
    REQUIRE(a.n_chunks <= 65535 && BQ <= 65535, CAKV_EUNSUPPORTED, "grid too large (B*Q=%lld)", (long long)BQ);
    return rc_from(cakv::launch_indexer_topk(a, BQ, fp8, workspace, reinterpret_cast<hipStream_t>(stream)));
}

size_t cakv_sparse_mqa_workspace(int64_t B, int64_t Q, int32_t H, int32_t D, int32_t K, int32_t n_win) {
    if (B < 0 || Q < 0 || H < 1 || D < 1 || K < 0 || n_win < 0) return 0;
    return attn_workspace(B * Q, H, D, (int64_t)K + n_win);
}

size_t cakv_dense_mqa_workspace(int64_t B, int64_t Q, int32_t H, int32_t D, int64_t N, int32_t n_win) {
    if (B < 0 || Q < 0 || H < 1 || D < 1 || N < 0 || n_win < 0) return 0;
    return attn_workspace(B * Q, H, D, N + n_win);
}

int cakv_sparse_mqa_fwd(const cakv_attn_params* p, const void* q, const void* kv_c, const int32_t* idx,
                        const void* kv_raw, const int32_t* raw_pos0, const int32_t* q_pos, const float* sinks,
                        int act_dtype, int64_t B, int64_t Q, int32_t H, int32_t D, int64_t N, int32_t K,
                        int64_t R, void* out, int out_dtype, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream) {
    int rc = check_attn_common(p, q, kv_c, kv_raw, raw_pos0, q_pos, sinks, act_dtype, B, Q, H, D, N, R, out,
                               out_dtype, lse);
    if (rc) return rc;
    REQUIRE(K >= 0 && K <= 65536, CAKV_EUNSUPPORTED, "K=%d out of 0..65536", K);
    if (B * Q == 0) return ok();
    if (K > 0) REQUIRE_PTR(idx, "idx");
    cakv::AttnArgs a{};
    fill_attn(a, p, q, kv_c, idx, kv_raw, raw_pos0, q_pos, sinks, Q, H, D, N, K, R, out, out_dtype, lse);
    // a non-NULL idx selects the sparse kernel; with K = 0 it never reads idx
    if (!a.idx) a.idx = q_pos;
    return run_attn(a, B * Q, H, D, (int64_t)K + p->n_win, act_dtype == CAKV_F32, workspace, workspace_bytes,
                    stream);
}

int cakv_dense_compressed_mqa_fwd(const cakv_attn_params* p, const void* q, const void* kv_c, const void* kv_raw,
                                  const int32_t* raw_pos0, const int32_t* q_pos, const float* sinks, int act_dtype,
                                  int64_t B, int64_t Q, int32_t H, int32_t D, int64_t N, int64_t R, void* out,
                                  int out_dtype, float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    int rc = check_attn_common(p, q, kv_c, kv_raw, raw_pos0, q_pos, sinks, act_dtype, B, Q, H, D, N, R, out,
                               out_dtype, lse);
    if (rc) return rc;
    REQUIRE(N <= 0x7fffffffLL, CAKV_EUNSUPPORTED, "N too large");
    if (B * Q == 0) return ok();
    cakv::AttnArgs a{};
    fill_attn(a, p, q, kv_c, nullptr, kv_raw, raw_pos0, q_pos, sinks, Q, H, D, N, 0, R, out, out_dtype, lse);
    return run_attn(a, B * Q, H, D, N + p->n_win, act_dtype == CAKV_F32, workspace, workspace_bytes, stream);
}

}  // extern "C"
