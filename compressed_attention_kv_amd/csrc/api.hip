// api.hip -- the C ABI of the compressed-attention library (include/cakv.h):
// argument validation, workspace sizing, launch geometry.  Every check runs
// before anything is enqueued; on error nothing is launched.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
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

// workspace one attention launch over BQ queries uses: the split partials
size_t attn_workspace(int64_t BQ, int32_t H, int32_t D, int64_t max_slots) {
    const int S = attn_splits(BQ, max_slots);
    if (S == 1) return 0;  // one split: the forward kernel writes the output itself
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return al((size_t)BQ * S * ((H + 1) / 2) * D * 4) + al((size_t)BQ * S * H * 2 * 4);
}

// what the *_workspace queries report: the largest launch workspace over
// every batch of 1 .. BQ queries, so that a workspace sized once for the
// largest batch serves every smaller one (the split count grows as the batch
// shrinks; beyond 256 queries there is one split and no partials)
size_t attn_workspace_query(int64_t BQ, int32_t H, int32_t D, int64_t max_slots) {
    size_t best = attn_workspace(BQ, H, D, max_slots);
    for (int64_t b = 1; b <= BQ && b <= 256; ++b) {
        const size_t w = attn_workspace(b, H, D, max_slots);
        if (w > best) best = w;
    }
    return best;
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
    REQUIRE(p->raw_ring == 0 || p->raw_ring == 1, CAKV_EINVAL, "raw_ring must be 0 or 1");
    if (p->raw_ring)
        REQUIRE(R >= p->n_win && R >= 1 && R <= 0x7fffffffLL, CAKV_EINVAL,
                "ring mode: the window ring needs R >= n_win rows (R=%lld, n_win=%d)", (long long)R, p->n_win);
    if (B * Q == 0) return CAKV_OK;
    REQUIRE_PTR(q, "q");
    if (!p->raw_ring) REQUIRE_PTR(raw_pos0, "raw_pos0");
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
    a.raw_ring = p->raw_ring;
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

int indexer_args(const void* q_idx, int q_dtype, const float* w, const void* k_idx, int k_dtype,
                 const float* k_scale, const int32_t* q_pos, int64_t B, int64_t Q, int64_t N, int32_t HI,
                 int32_t dI, int32_t m, int32_t k, int32_t* idx, cakv::IndexerArgs& a, bool& fp8_mode,
                 bool& empty);

// workspace of an attention backward launch over BQ queries, and what the
// query reports (the largest over every batch of 1 .. BQ queries)
size_t bwd_workspace(int64_t BQ, int32_t H, int64_t max_slots) {
    return cakv::mqa_bwd_workspace_bytes(BQ, H, max_slots, attn_splits(BQ, max_slots));
}
size_t bwd_workspace_query(int64_t BQ, int32_t H, int64_t max_slots) {
    size_t best = bwd_workspace(BQ, H, max_slots);
    for (int64_t b = 1; b <= BQ && b <= 256; ++b) {
        const size_t w = bwd_workspace(b, H, max_slots);
        if (w > best) best = w;
    }
    return best;
}

// The allocation-free indexer call keeps its workspace here: one copy of the
// array per GPU, held until the process ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept per device.
constexpr size_t kScratchBytes = CAKV_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(CAKV_ELAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
    REQUIRE(dev >= 0 && dev < kMaxDevices, CAKV_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(CAKV_ELAUNCH, "hipGetSymbolAddress of the static scratch failed on device %d: %s", dev,
                        hipGetErrorString(e));
        REQUIRE((reinterpret_cast<uintptr_t>(p) & 255u) == 0, CAKV_ELAUNCH, "static scratch is not 256-byte aligned");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CAKV_OK;
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
    REQUIRE(m >= 1 && m <= 4096, CAKV_EUNSUPPORTED, "m=%d out of 1..4096", m);
    return cakv_kv_compress_ex(x, x_dtype, gate, 0, B, T, D, m, m, out, out_dtype, out_scale, stream);
}

int cakv_kv_compress_ex(const void* x, int x_dtype, const float* gate, int gate_per_channel, int64_t B,
                        int64_t T, int64_t D, int32_t m, int32_t span, void* out, int out_dtype, float* out_scale,
                        void* stream) {
    REQUIRE(B >= 0 && T >= 0, CAKV_EINVAL, "negative size (B=%lld T=%lld)", (long long)B, (long long)T);
    REQUIRE(m >= 1 && m <= 4096, CAKV_EUNSUPPORTED, "m=%d out of 1..4096", m);
    REQUIRE(span >= m && span <= 8192, CAKV_EUNSUPPORTED, "span=%d: m <= span <= 8192 (m=%d)", span, m);
    REQUIRE(gate_per_channel == 0 || gate_per_channel == 1, CAKV_EINVAL, "gate_per_channel must be 0 or 1");
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
    return rc_from(cakv::launch_kv_compress(x, x_dtype, gate, gate_per_channel != 0, B, T, D, m, span, out,
                                            out_dtype, out_scale, reinterpret_cast<hipStream_t>(stream)));
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

// Validates one append and fills its kernel arguments and the batch kernel's
// kind code (4 * activations bf16 + 2 * cache fp8 + per-channel gates);
// empty is set when there is nothing to do (B == 0).
static int append_args(const void* x_tok, const float* gate_tok, int gate_per_channel, const int32_t* pos,
                       int act_dtype, int64_t B, int64_t D, void* raw_ring, float* gate_ring, int64_t Rr,
                       void* win_ring, int64_t Rw, void* cache, int cache_dtype, float* cache_scale, int64_t N,
                       int32_t m, int32_t span, const cakv_prep_params* prep, cakv::AppendArgs& a, int32_t& kind,
                       bool& empty) {
    empty = false;
    REQUIRE(B >= 0 && N >= 0, CAKV_EINVAL, "negative size (B=%lld N=%lld)", (long long)B, (long long)N);
    REQUIRE(act_dtype == CAKV_F32 || act_dtype == CAKV_BF16, CAKV_EINVAL, "act_dtype must be F32 or BF16");
    REQUIRE(cache_dtype == act_dtype || cache_dtype == CAKV_FP8_E4M3, CAKV_EINVAL,
            "cache_dtype must be act_dtype or FP8_E4M3");
    REQUIRE(gate_per_channel == 0 || gate_per_channel == 1, CAKV_EINVAL, "gate_per_channel must be 0 or 1");
    REQUIRE(D >= 8 && D <= 4096 && D % 8 == 0, CAKV_EUNSUPPORTED, "D=%lld: 8..4096, a multiple of 8", (long long)D);
    REQUIRE(m >= 1 && m <= 4096, CAKV_EUNSUPPORTED, "m=%d out of 1..4096", m);
    REQUIRE(span >= m && span <= 8192, CAKV_EUNSUPPORTED, "span=%d: m <= span <= 8192 (m=%d)", span, m);
    REQUIRE(Rr >= span && Rr <= 0x7fffffffLL, CAKV_EINVAL,
            "raw ring of %lld rows: at least span=%d (the compressor reads the span's earlier tokens from it)",
            (long long)Rr, span);
    REQUIRE((cache_dtype == CAKV_FP8_E4M3) == (cache_scale != nullptr), CAKV_EINVAL,
            "cache_scale is required for an FP8_E4M3 cache and must be NULL otherwise");
    REQUIRE(!(prep && cache_dtype == CAKV_FP8_E4M3), CAKV_EINVAL, "fp8 caches hold unprepared entries: prep must be NULL");
    REQUIRE(!win_ring || prep, CAKV_EINVAL, "a window ring holds prepared rows: prep is required");
    if (win_ring) REQUIRE(Rw >= 1 && Rw <= 0x7fffffffLL, CAKV_EINVAL, "window ring rows Rw=%lld", (long long)Rw);
    if (prep) {
        REQUIRE(prep->rope_dims >= 0 && (prep->rope_dims & 1) == 0 && prep->rope_dims <= D, CAKV_EINVAL,
                "rope_dims=%d: even, 0..D", prep->rope_dims);
        REQUIRE(prep->rope_base > 0.0f && isfinite(prep->rope_base), CAKV_EINVAL, "rope_base must be positive");
        REQUIRE(prep->rms_eps >= 0.0f && isfinite(prep->rms_eps), CAKV_EINVAL, "rms_eps must be >= 0");
        REQUIRE((N - 1) * (int64_t)m + prep->entry_pos_offset <= 0x7fffffffLL &&
                    prep->entry_pos_offset >= -0x7fffffffLL,
                CAKV_EINVAL, "entry positions must fit in int32");
        if (prep->gamma_kv) REQUIRE(aligned16(prep->gamma_kv), CAKV_EINVAL, "gamma_kv must be 16-byte aligned");
    }
    if (B == 0) {
        empty = true;
        return ok();
    }
    REQUIRE(B <= 0x7fffffffLL, CAKV_EUNSUPPORTED, "B too large");
    REQUIRE_PTR(x_tok, "x_tok");
    REQUIRE_PTR(gate_tok, "gate_tok");
    REQUIRE_PTR(pos, "pos");
    REQUIRE_PTR(raw_ring, "raw_ring");
    REQUIRE_PTR(gate_ring, "gate_ring");
    if (win_ring) REQUIRE(aligned16(win_ring), CAKV_EINVAL, "win_ring must be 16-byte aligned");
    if (N > 0) REQUIRE_PTR(cache, "cache");
    if (cache_scale) REQUIRE(aligned16(cache_scale), CAKV_EINVAL, "cache_scale must be 16-byte aligned");
    a = cakv::AppendArgs{};
    a.x_tok = x_tok;
    a.gate_tok = gate_tok;
    a.pos = pos;
    a.raw_ring = raw_ring;
    a.gate_ring = gate_ring;
    a.win_ring = win_ring;
    a.cache = cache;
    a.cache_scale = cache_scale;
    a.Rr = Rr;
    a.Rw = win_ring ? Rw : 1;
    a.N = N;
    a.D = (int32_t)D;
    a.m = m;
    a.span = span;
    a.prep = prep != nullptr;
    if (prep) {
        a.gamma_kv = prep->gamma_kv;
        a.rope_dims = prep->rope_dims;
        a.pos_off = prep->entry_pos_offset;
        a.eps = prep->rms_eps;
        a.rope_ratio = cakv::rope_ratio_of(prep->rope_base, prep->rope_dims);
    }
    kind = 4 * (act_dtype == CAKV_BF16 ? 1 : 0) + 2 * (cache_dtype == CAKV_FP8_E4M3 ? 1 : 0) +
           (gate_per_channel != 0 ? 1 : 0);
    return ok();
}

int cakv_kv_append(const void* x_tok, const float* gate_tok, int gate_per_channel, const int32_t* pos,
                   int act_dtype, int64_t B, int64_t D, void* raw_ring, float* gate_ring, int64_t Rr,
                   void* win_ring, int64_t Rw, void* cache, int cache_dtype, float* cache_scale, int64_t N,
                   int32_t m, int32_t span, const cakv_prep_params* prep, void* stream) {
    cakv::AppendArgs a;
    int32_t kind = 0;
    bool empty = false;
    const int rc = append_args(x_tok, gate_tok, gate_per_channel, pos, act_dtype, B, D, raw_ring, gate_ring, Rr,
                               win_ring, Rw, cache, cache_dtype, cache_scale, N, m, span, prep, a, kind, empty);
    if (rc || empty) return rc;
    return rc_from(cakv::launch_kv_append(a, B, act_dtype, cache_dtype, gate_per_channel != 0,
                                          reinterpret_cast<hipStream_t>(stream)));
}

int cakv_kv_append_batch(const cakv_append_call* calls, int32_t n, const int32_t* pos, int64_t B, void* stream) {
    static_assert(CAKV_APPEND_BATCH_MAX == cakv::kAppendBatchMax, "batch size of the header and the kernel");
    REQUIRE(calls, CAKV_EINVAL, "calls must not be NULL");
    REQUIRE(n >= 1 && n <= CAKV_APPEND_BATCH_MAX, CAKV_EINVAL, "n=%d: 1 .. %d appends per batch", n,
            CAKV_APPEND_BATCH_MAX);
    cakv::AppendBatch ab{};
    bool empty = false;
    for (int i = 0; i < n; ++i) {
        const cakv_append_call& c = calls[i];
        const int rc = append_args(c.x_tok, c.gate_tok, c.gate_per_channel, pos, c.act_dtype, B, c.D, c.raw_ring,
                                   c.gate_ring, c.Rr, c.win_ring, c.Rw, c.cache, c.cache_dtype, c.cache_scale, c.N,
                                   c.m, c.span, c.prep, ab.a[i], ab.kind[i], empty);
        if (rc) return rc;
        // the appends run concurrently: no two may write the same buffer
        // (with no tokens nothing runs, and the buffers may be NULL)
        for (int k = 0; k < i && !empty; ++k) {
            const cakv_append_call& o = calls[k];
            REQUIRE(c.raw_ring != o.raw_ring && c.gate_ring != o.gate_ring &&
                        (!c.win_ring || c.win_ring != o.win_ring) && (!c.cache || c.cache != o.cache) &&
                        (!c.cache_scale || c.cache_scale != o.cache_scale),
                    CAKV_EINVAL, "appends %d and %d of a batch write the same buffer", k, i);
        }
    }
    if (empty) return ok();
    return rc_from(cakv::launch_kv_append_batch(ab, n, B, reinterpret_cast<hipStream_t>(stream)));
}

size_t cakv_indexer_topk_workspace(int64_t B, int64_t Q, int64_t N, int32_t k) {
    if (B < 0 || Q < 0 || N < 0 || k < 1) return 0;
    return cakv::indexer_workspace_bytes(B, Q, N, k);
}

int cakv_indexer_topk(const void* q_idx, int q_dtype, const float* w, const void* k_idx, int k_dtype,
                      const float* k_scale, const int32_t* q_pos, int64_t B, int64_t Q, int64_t N,
                      int32_t HI, int32_t dI, int32_t m, int32_t k, int32_t* idx, void* workspace,
                      size_t workspace_bytes, void* stream) {
    cakv::IndexerArgs a{};
    bool fp8 = false, empty = false;
    int rc = indexer_args(q_idx, q_dtype, w, k_idx, k_dtype, k_scale, q_pos, B, Q, N, HI, dI, m, k, idx, a, fp8,
                          empty);
    if (rc || empty) return rc;
    const int64_t BQ = B * Q;
    const size_t need = cakv::indexer_workspace_bytes(B, Q, N, k);
    REQUIRE(workspace_bytes >= need, CAKV_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    REQUIRE(workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, CAKV_EWORKSPACE,
            "workspace must be non-NULL and 256-byte aligned");
    return rc_from(cakv::launch_indexer_topk(a, BQ, fp8, workspace, reinterpret_cast<hipStream_t>(stream)));
}

int cakv_indexer_topk_noalloc(const void* q_idx, int q_dtype, const float* w, const void* k_idx, int k_dtype,
                              const float* k_scale, const int32_t* q_pos, int64_t B, int64_t Q, int64_t N,
                              int32_t HI, int32_t dI, int32_t m, int32_t k, int32_t* idx, void* stream) {
    cakv::IndexerArgs a{};
    bool fp8 = false, empty = false;
    int rc = indexer_args(q_idx, q_dtype, w, k_idx, k_dtype, k_scale, q_pos, B, Q, N, HI, dI, m, k, idx, a, fp8,
                          empty);
    if (rc || empty) return rc;
    const int64_t BQ = B * Q;
    const size_t need = cakv::indexer_workspace_bytes(B, Q, N, k);
    REQUIRE(need <= kScratchBytes, CAKV_EWORKSPACE,
            "B*Q=%lld queries over N=%lld entries need %zu bytes of scratch, more than the %zu bytes the "
            "allocation-free call holds per GPU; use cakv_indexer_topk with a workspace",
            (long long)BQ, (long long)N, need, kScratchBytes);
    void* ws = nullptr;
    rc = scratch_of_current_device(&ws);
    if (rc) return rc;
    return rc_from(cakv::launch_indexer_topk(a, BQ, fp8, ws, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Validation of an indexer call and its launch arguments (shared by the
// workspace and the allocation-free entry points).  `empty`: nothing to do.
int indexer_args(const void* q_idx, int q_dtype, const float* w, const void* k_idx, int k_dtype,
                 const float* k_scale, const int32_t* q_pos, int64_t B, int64_t Q, int64_t N, int32_t HI,
                 int32_t dI, int32_t m, int32_t k, int32_t* idx, cakv::IndexerArgs& a, bool& fp8_mode,
                 bool& empty) {
    empty = false;
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
    fp8_mode = fp8;
    const int64_t BQ = B * Q;
    if (BQ == 0) {
        empty = true;
        return ok();
    }
    REQUIRE(BQ <= 0x7fffffffLL, CAKV_EUNSUPPORTED, "B*Q too large");
    REQUIRE_PTR(q_idx, "q_idx");
    REQUIRE_PTR(w, "w");
    REQUIRE_PTR(q_pos, "q_pos");
    REQUIRE_PTR(idx, "idx");
    if (N > 0) {
        REQUIRE_PTR(k_idx, "k_idx");
        if (fp8) REQUIRE_PTR(k_scale, "k_scale");
    }
    a = cakv::IndexerArgs{};
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
    return CAKV_OK;
}

}  // namespace

extern "C" {

size_t cakv_mqa_bwd_workspace(int64_t B, int64_t Q, int32_t H, int32_t D, int64_t n_keys, int32_t n_win) {
    if (B < 0 || Q < 0 || H < 1 || D < 1 || n_keys < 0 || n_win < 0) return 0;
    return bwd_workspace_query(B * Q, H, n_keys + n_win);
}

int cakv_mqa_bwd(const cakv_attn_params* p, const void* q, const void* kv_c, const int32_t* idx, const void* kv_raw,
                 const int32_t* raw_pos0, const int32_t* q_pos, const float* sinks, int act_dtype, int64_t B, int64_t Q,
                 int32_t H, int32_t D, int64_t N, int32_t K, int64_t R, const void* out, int out_dtype,
                 const float* lse, const float* dout, float* dq, float* dkv_c, float* dkv_raw, float* dsinks,
                 float* dgamma_q, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_attn_common(p, q, kv_c, kv_raw, raw_pos0, q_pos, sinks, act_dtype, B, Q, H, D, N, R,
                               const_cast<void*>(out), out_dtype, const_cast<float*>(lse));
    if (rc) return rc;
    REQUIRE(D == 512 && act_dtype == CAKV_BF16, CAKV_EUNSUPPORTED,
            "backward: bf16 activations with D = 512 (D=%d)", D);
    if (idx) REQUIRE(K >= 0 && K <= 65536, CAKV_EUNSUPPORTED, "K=%d out of 0..65536", K);
    REQUIRE(N <= 0x7fffffffLL, CAKV_EUNSUPPORTED, "N too large");
    if (B * Q == 0) return ok();
    REQUIRE_PTR(out, "out");
    REQUIRE_PTR(lse, "lse");
    REQUIRE_PTR(dout, "dout");
    REQUIRE_PTR(dq, "dq");
    if (N > 0) REQUIRE_PTR(dkv_c, "dkv_c");
    if (R > 0) REQUIRE_PTR(dkv_raw, "dkv_raw");
    if (dsinks) REQUIRE(aligned16(dsinks), CAKV_EINVAL, "dsinks must be 16-byte aligned");
    if (dgamma_q) REQUIRE(aligned16(dgamma_q), CAKV_EINVAL, "dgamma_q must be 16-byte aligned");
    const int64_t BQ = B * Q;
    REQUIRE(BQ <= 65535, CAKV_EUNSUPPORTED, "backward: B*Q=%lld above 65535", (long long)BQ);
    const int64_t max_slots = (idx ? (int64_t)K : N) + p->n_win;
    const size_t need = bwd_workspace(BQ, H, max_slots);
    REQUIRE(workspace_bytes >= need, CAKV_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    REQUIRE(workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, CAKV_EWORKSPACE,
            "workspace must be non-NULL and 256-byte aligned");
    cakv::BwdArgs w{};
    fill_attn(w.f, p, q, kv_c, idx, kv_raw, raw_pos0, q_pos, sinks, Q, H, D, N, idx ? K : 0, R,
              const_cast<void*>(out), out_dtype, const_cast<float*>(lse));
    w.f.n_splits = attn_splits(BQ, max_slots);
    w.out = out;
    w.out_f32 = out_dtype == CAKV_F32;
    // one query per sequence: the selected entries of a query are distinct
    // (a precondition) and sequences share no rows, so every key row is
    // touched by one workgroup only
    w.unique_rows = Q == 1;
    w.lse = lse;
    w.dout = dout;
    w.dq = dq;
    w.dkv_c = dkv_c;
    w.dkv_raw = dkv_raw;
    w.dsinks = dsinks;
    w.dgamma_q = dgamma_q;
    w.tau = p->softmax_scale > 0.0f ? p->softmax_scale : (float)(1.0 / sqrt((double)D));
    return rc_from(cakv::launch_mqa_bwd(w, BQ, max_slots, workspace, reinterpret_cast<hipStream_t>(stream)));
}

int cakv_kv_prepare_bwd(const void* kv_in, int act_dtype, const float* dy, float* dx, float* dgamma_kv, int64_t B,
                        int64_t N, int64_t D, int64_t j0, int64_t n, const float* gamma_kv, int32_t m,
                        int32_t rope_dims, float rope_base, int32_t entry_pos_offset, float rms_eps, void* stream) {
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
    REQUIRE_PTR(dy, "dy");
    REQUIRE_PTR(dx, "dx");
    if (gamma_kv) REQUIRE(aligned16(gamma_kv), CAKV_EINVAL, "gamma_kv must be 16-byte aligned");
    if (dgamma_kv) REQUIRE(aligned16(dgamma_kv), CAKV_EINVAL, "dgamma_kv must be 16-byte aligned");
    return rc_from(cakv::launch_kv_prepare_bwd(kv_in, dy, dx, dgamma_kv, act_dtype == CAKV_F32 ? 0 : 1, B, N, D, j0,
                                               n, gamma_kv, m, rope_dims, cakv::rope_ratio_of(rope_base, rope_dims),
                                               entry_pos_offset, rms_eps, reinterpret_cast<hipStream_t>(stream)));
}

size_t cakv_kv_compress_bwd_workspace(int64_t B, int64_t T, int64_t D, int32_t m) {
    if (B < 0 || T < 0 || D < 1 || m < 1) return 0;
    return cakv::kv_compress_bwd_workspace_bytes(B, T, D, m);
}

int cakv_kv_compress_bwd(const void* x, int x_dtype, const float* gate, int gate_per_channel, int64_t B, int64_t T,
                         int64_t D, int32_t m, int32_t span, const float* dc, float* dx, float* dgate, void* workspace,
                         size_t workspace_bytes, void* stream) {
    REQUIRE(B >= 0 && T >= 0, CAKV_EINVAL, "negative size (B=%lld T=%lld)", (long long)B, (long long)T);
    REQUIRE(m >= 1 && m <= 4096, CAKV_EUNSUPPORTED, "m=%d out of 1..4096", m);
    REQUIRE(span >= m && span <= 8192, CAKV_EUNSUPPORTED, "span=%d: m <= span <= 8192 (m=%d)", span, m);
    REQUIRE(gate_per_channel == 0 || gate_per_channel == 1, CAKV_EINVAL, "gate_per_channel must be 0 or 1");
    REQUIRE(D >= 4 && D <= 4096 && D % 4 == 0, CAKV_EUNSUPPORTED, "D=%lld: 4..4096, a multiple of 4", (long long)D);
    REQUIRE(x_dtype == CAKV_F32 || x_dtype == CAKV_BF16, CAKV_EINVAL, "x_dtype must be F32 or BF16");
    if (B * T == 0) return ok();
    REQUIRE_PTR(x, "x");
    REQUIRE_PTR(gate, "gate");
    REQUIRE_PTR(dx, "dx");
    REQUIRE_PTR(dgate, "dgate");
    if (T / m > 0) REQUIRE_PTR(dc, "dc");
    const size_t need = cakv::kv_compress_bwd_workspace_bytes(B, T, D, m);
    REQUIRE(workspace_bytes >= need, CAKV_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    if (need) REQUIRE(workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, CAKV_EWORKSPACE,
                      "workspace must be non-NULL and 256-byte aligned");
    return rc_from(cakv::launch_kv_compress_bwd(x, x_dtype, gate, gate_per_channel != 0, B, T, D, m, span, dc, dx,
                                                dgate, workspace, reinterpret_cast<hipStream_t>(stream)));
}

int cakv_indexer_bwd(const void* q_idx, int q_dtype, const float* w, const void* k_idx, int k_dtype,
                     const float* k_scale, const int32_t* q_pos, const int32_t* idx, const float* dS, int64_t B,
                     int64_t Q, int64_t N, int32_t HI, int32_t dI, int32_t m, int32_t K, float* dq_idx, float* dw,
                     float* dk, void* stream) {
    REQUIRE(B >= 0 && Q >= 0 && N >= 0, CAKV_EINVAL, "negative size");
    REQUIRE(m >= 1, CAKV_EINVAL, "m=%d must be >= 1", m);
    REQUIRE(K >= 0 && K <= 65536, CAKV_EUNSUPPORTED, "K=%d out of 0..65536", K);
    REQUIRE(N <= 0x7fffffffLL, CAKV_EUNSUPPORTED, "N too large");
    const bool f32 = q_dtype == CAKV_F32 && k_dtype == CAKV_F32;
    const bool fp8 = q_dtype == CAKV_BF16 && k_dtype == CAKV_FP8_E4M3;
    REQUIRE(f32 || fp8, CAKV_EUNSUPPORTED, "dtypes: (F32 q, F32 k) or (BF16 q, FP8_E4M3 k)");
    REQUIRE(HI >= 1 && HI <= 64 && dI >= 8 && dI <= 128 && dI % 8 == 0, CAKV_EUNSUPPORTED,
            "HI <= 64, dI a multiple of 8 up to 128 (HI=%d dI=%d)", HI, dI);
    REQUIRE(fp8 == (k_scale != nullptr), CAKV_EINVAL, "k_scale is required for FP8_E4M3 keys and NULL otherwise");
    const int64_t BQ = B * Q;
    if (BQ == 0) return ok();
    REQUIRE(BQ < (1LL << 23), CAKV_EUNSUPPORTED, "B*Q=%lld must be below 2^23", (long long)BQ);
    REQUIRE_PTR(q_idx, "q_idx");
    REQUIRE_PTR(w, "w");
    REQUIRE_PTR(q_pos, "q_pos");
    REQUIRE_PTR(dq_idx, "dq_idx");
    REQUIRE_PTR(dw, "dw");
    if (K > 0) {
        REQUIRE_PTR(idx, "idx");
        REQUIRE_PTR(dS, "dS");
    }
    if (N > 0) {
        REQUIRE_PTR(k_idx, "k_idx");
        REQUIRE_PTR(dk, "dk");
        if (fp8) REQUIRE_PTR(k_scale, "k_scale");
    }
    cakv::IndexerBwdArgs a{};
    a.q_idx = q_idx;
    a.w = w;
    a.k_idx = k_idx;
    a.k_scale = k_scale;
    a.q_pos = q_pos;
    a.idx = idx;
    a.dS = dS;
    a.dq = dq_idx;
    a.dw = dw;
    a.dk = dk;
    a.Q = Q;
    a.N = N;
    a.HI = HI;
    a.dI = dI;
    a.m = m;
    a.K = K;
    return rc_from(cakv::launch_indexer_bwd(a, BQ, f32, fp8, reinterpret_cast<hipStream_t>(stream)));
}

size_t cakv_sparse_mqa_workspace(int64_t B, int64_t Q, int32_t H, int32_t D, int32_t K, int32_t n_win) {
    if (B < 0 || Q < 0 || H < 1 || D < 1 || K < 0 || n_win < 0) return 0;
    return attn_workspace_query(B * Q, H, D, (int64_t)K + n_win);
}

size_t cakv_dense_mqa_workspace(int64_t B, int64_t Q, int32_t H, int32_t D, int64_t N, int32_t n_win) {
    if (B < 0 || Q < 0 || H < 1 || D < 1 || N < 0 || n_win < 0) return 0;
    return attn_workspace_query(B * Q, H, D, N + n_win);
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
