/*
 * cakv.h -- C ABI of the MI355X (gfx950) compressed-attention library:
 * the hot path of DeepSeek-V4's hybrid attention, CSA (compressed sparse
 * attention) and HCA (heavily compressed attention).
 *
 * Pages the operations follow (cited by short name):
 *   [V4-Pro card]  "DeepSeek V4-Pro", llm-arch-kb (lizeman.github.io),
 *                  "What's new in V4", item 1 "Hybrid attention".
 *   [V4 digest]    DeepSeek V4 technical-report digest (agentupdate.ai),
 *                  hybrid-attention section: the four CSA steps and the HCA
 *                  paragraph.
 *   [Visualised]   "DeepSeek V4-Pro Architecture: KV Cache Compression and
 *                  Hyper-Connections Visualised" (webconsulting.at),
 *                  "Key points" and "Dual Compression and Indexing".
 *
 * Conventions shared by every call
 *   - All tensors are dense, row-major, innermost dimension contiguous, on
 *     the current HIP device.  Pointers are device pointers unless stated.
 *     Every pointer must be 16-byte aligned.
 *   - The caller owns every buffer (inputs, outputs, workspace).  The library
 *     allocates nothing, keeps no pointer after returning and never
 *     synchronises: work is enqueued on `stream` (a hipStream_t, NULL for the
 *     default stream) and runs asynchronously.
 *   - Return value: CAKV_OK (0) or a negative error code.  Every argument is
 *     validated on the host before anything is enqueued, so on error nothing
 *     runs; cakv_last_error() then names the argument (thread-local string).
 *   - Values read on the device (positions, indices) are clamped for memory
 *     safety as documented per call; they are never a cause of an error code.
 *   - Results are deterministic: the same inputs and sizes give bitwise-equal
 *     outputs run to run.
 *
 * Positions and visibility (shared by the attention calls and the indexer)
 *   A query at absolute position t sees compressed entry j of a cache built
 *   with ratio m iff the whole block of entry j precedes it: j < floor(t/m)
 *   (and j < N, the number of entries the cache holds).  The raw sliding
 *   window of a query at t is the positions max(0, t - n_win + 1) .. t,
 *   its own token included [V4-Pro card: window of n_win uncompressed
 *   entries on every CSA/HCA layer, because compressed keys cannot reach
 *   inside the current block].
 */
#ifndef CAKV_H
#define CAKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* error codes */
#define CAKV_OK 0
#define CAKV_EINVAL (-1)      /* bad argument: NULL, size, alignment, dtype mismatch */
#define CAKV_EUNSUPPORTED (-2) /* valid but not implemented: head dim, ratio, k, ... */
#define CAKV_EWORKSPACE (-3)  /* workspace missing or smaller than the *_workspace query */
#define CAKV_ELAUNCH (-4)     /* the HIP runtime refused a launch */

/* element types */
#define CAKV_F32 0
#define CAKV_BF16 1
#define CAKV_FP8_E4M3 2 /* OCP E4M3 ("E4M3FN"): bias 7, max 448, S.1111.111 = NaN */

/* Library version: major*10000 + minor*100 + patch. */
int cakv_version(void);

/* Message describing the last error returned on this thread ("" if none). */
const char* cakv_last_error(void);

/* Profiling aid (not part of the method): for the next n launches, made by
 * calls on the calling thread, of the kernel whose function name is `kernel`
 * (one of kv_compress_kernel, idx_zero_kernel, idx_score_fp8_kernel,
 * idx_score_f32_kernel, idx_refine_kernel, idx_select_kernel, mqa_fwd_kernel,
 * mqa_combine_kernel), record starts[i] on the call's stream just before the
 * i-th such launch and ends[i] just after it.  The events are hipEvent_t
 * handles created and owned by the caller; the library copies the n handles
 * and keeps them until the n launches have happened or the next call of this
 * function (n = 0 or kernel = NULL clears them).  Results are unaffected.
 * Errors: EINVAL (n < 0, or a NULL array or event with n > 0). */
int cakv_profile_kernel_events(const char* kernel, void* const* starts, void* const* ends, int n);

/* ---------------------------------------------------------------------------
 * kv_compress  [V4 digest, CSA step 1 and HCA paragraph; V4-Pro card: CSA
 * compresses every m=4 tokens, HCA every m'=128, into one KV entry;
 * Visualised: learned weighted averages]
 *
 * For each sequence b and each whole block j < floor(T/m):
 *     a = softmax(gate[b, j*m .. j*m+m-1]);   out[b, j, :] = sum_i a_i x[b, j*m+i, :]
 * Blocks do not overlap; a trailing partial block produces no entry (its
 * tokens stay in the raw window).
 *   x        [B, T, D]   x_dtype  CAKV_F32 or CAKV_BF16
 *   gate     [B, T]      float32 gate logits (finite)
 *   m        1 .. 4096
 *   out      [B, floor(T/m), D]  out_dtype CAKV_F32, CAKV_BF16 (round to nearest
 *            even) or CAKV_FP8_E4M3 (one byte per element)
 *   out_scale [B, floor(T/m)] float32, required for CAKV_FP8_E4M3 and NULL
 *            otherwise.  fp8 mode stores a power-of-two scale s = 2^e per
 *            entry, e the smallest integer >= -126 with max_d |c_d| <= 448 * 2^e
 *            (e = 0 for an all-zero entry), and codes E4M3(c_d / s) rounded to
 *            nearest even; the dequantised value is code * s.
 *   D        1 .. 4096, a multiple of 4 (of 8 for bf16 input)
 * Errors: EINVAL (NULL pointers, sizes, dtypes), EUNSUPPORTED (m, D).
 * ------------------------------------------------------------------------- */
int cakv_kv_compress(const void* x, int x_dtype, const float* gate, int64_t B, int64_t T,
                     int64_t D, int32_t m, void* out, int out_dtype, float* out_scale,
                     void* stream);

/* ---------------------------------------------------------------------------
 * kv_prepare  [V4-Pro card, "Hybrid attention": RMSNorm on the single
 * compressed KV head before the attention dot product; RoPE on the last 64
 * dims of each KV entry]
 *
 * The key (= value) vector of compressed entries j0 .. j0+n-1 of each of the B
 * sequences:
 *     y = gamma_kv * c / sqrt(mean_d(c_d^2) + rms_eps),
 * then the last rope_dims channels, in consecutive pairs (2i, 2i+1) counted
 * from D - rope_dims, rotated by the angle pi * rope_base^(-2i/rope_dims) with
 * pi = j*m + entry_pos_offset, the entry's position.  The attention calls
 * read compressed entries in this form: run it once on every entry when the
 * entry enters the cache (after kv_compress), not per attention call.
 *   kv_in   [B, N, D]  act_dtype CAKV_F32 or CAKV_BF16, raw entries c
 *   kv_out  [B, N, D]  same dtype; only entries j0 .. j0+n-1 are written
 *           (bf16: round to nearest even).  kv_out == kv_in works in place;
 *           other overlaps are undefined.
 *   gamma_kv [D] float32 device pointer, NULL = all ones
 *   D        8 .. 4096, a multiple of 8; rope_dims even, 0 .. D
 * Arithmetic in fp32.  Errors: EINVAL (NULL pointers, alignment, ranges,
 * positions beyond int32), EUNSUPPORTED (D).
 * ------------------------------------------------------------------------- */
int cakv_kv_prepare(const void* kv_in, void* kv_out, int act_dtype, int64_t B, int64_t N, int64_t D,
                    int64_t j0, int64_t n, const float* gamma_kv, int32_t m, int32_t rope_dims,
                    float rope_base, int32_t entry_pos_offset, float rms_eps, void* stream);

/* ---------------------------------------------------------------------------
 * indexer_topk  [V4 digest, CSA step 2: a light indexer scores every
 * compressed entry for each query and keeps the top k; V4-Pro card: 64
 * Lightning-Indexer heads of dim 128 select k=1024 entries; Visualised:
 * low-precision similarity pass over ~262,000 entries keeps 1,024]
 *
 * For query (b, i) at position t = q_pos[b, i], over visible entries
 * j < n_vis = min(floor(t/m), N):
 *     S(j) = sum_h w[b,i,h] * ReLU(q_idx[b,i,h,:] . k_idx[b,j,:])
 * keeps the first min(k, n_vis) entries under (S descending, j ascending),
 * writes them ascending by j and pads with -1 up to k.
 *   q_idx  [B, Q, HI, dI]  q_dtype     CAKV_F32 or CAKV_BF16
 *   w      [B, Q, HI]      float32
 *   k_idx  [B, N, dI]      k_dtype     CAKV_F32 or CAKV_FP8_E4M3
 *   k_scale [B, N]         float32 per-entry scale for fp8 keys (the key is
 *                          code * scale), NULL for f32 keys
 *   q_pos  [B, Q]          int32 positions (negative values are treated as 0)
 *   idx    [B, Q, k]       int32 output
 * Modes: q f32 + k f32 computes every S(j) in fp32 with fmaf chains, head dim
 * ascending then heads ascending (bit-exact with a plain CPU loop in that
 * order); q bf16 + k fp8 computes the dot products on bf16 matrix cores with
 * fp32 accumulation (keys are decoded exactly; summation order differs).
 * Inputs must be finite.  HI <= 64 (bf16 mode: HI a multiple of 32 up to 64,
 * dI a multiple of 32 up to 256), k 1 .. 4096.
 * Workspace: at least cakv_indexer_topk_workspace(B, Q, N, k) bytes, 256-byte
 * aligned; its contents on entry do not matter.
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE.
 * ------------------------------------------------------------------------- */
size_t cakv_indexer_topk_workspace(int64_t B, int64_t Q, int64_t N, int32_t k);
int cakv_indexer_topk(const void* q_idx, int q_dtype, const float* w, const void* k_idx,
                      int k_dtype, const float* k_scale, const int32_t* q_pos, int64_t B,
                      int64_t Q, int64_t N, int32_t HI, int32_t dI, int32_t m, int32_t k,
                      int32_t* idx, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Attention parameters shared by sparse_mqa_fwd and dense_compressed_mqa_fwd.
 * [V4-Pro card: RMSNorm on each query head and on the single compressed KV
 * head before the dot product; RoPE on the last 64 dims of query, KV entry and
 * core-attention output, the output rotated back; learnable per-head sink
 * logits added to the softmax denominator]
 * ------------------------------------------------------------------------- */
typedef struct cakv_attn_params {
    int32_t m;                /* compression ratio of kv_c (visibility) */
    int32_t n_win;            /* raw window length, 0 .. 4096 */
    int32_t rope_dims;        /* r: rotated trailing dims, even, 0 .. D */
    float rope_base;          /* theta_i = rope_base^(-2i/r) */
    float softmax_scale;      /* 0 selects 1/sqrt(D) */
    float rms_eps;            /* RMSNorm epsilon of the query heads */
    const float* gamma_q;     /* [D] device pointer, NULL = all ones */
} cakv_attn_params;

/* ---------------------------------------------------------------------------
 * sparse_mqa_fwd  [V4 digest, CSA step 3: multi-query attention over the
 * selected compressed entries; V4-Pro card: shared-KV MQA, 128 heads of dim
 * 512, plus the raw window and the sink]
 *
 * Query (b, i, h) at t = q_pos[b, i] attends, in one softmax, to
 *   - compressed entries idx[b, i, s] (s < K) that are >= 0 and visible,
 *   - raw window rows at positions max(0, t-n_win+1) .. t that lie inside
 *     [raw_pos0[b], raw_pos0[b] + R) (kv_raw row p - raw_pos0[b]),
 *   - the sink: exp(sinks[h]) added to the denominator with a zero value.
 * Keys and values are the same vector k_hat = RoPE_pi(gamma_kv * v / rms(v)),
 * pi the key's position; the query is RoPE_t(gamma_q * q / rms(q)); logits are
 * softmax_scale * (q_hat . k_hat).  The output is rotated back by -t.
 * Every key row is read as cakv_kv_prepare left it (already k_hat: a key
 * depends only on its own entry or token and its position, so it is prepared
 * once, when written): kv_c entry j prepared at j*m + offset, and kv_raw row r
 * of sequence b prepared at position raw_pos0[b] + r (cakv_kv_prepare with
 * m = 1 and entry_pos_offset = raw_pos0[b] on that sequence's rows).
 *   q       [B, Q, H, D]  act_dtype   CAKV_BF16 or CAKV_F32 (also kv_c, kv_raw)
 *   kv_c    [B, N, D]     compressed cache (ratio p->m), prepared entries
 *   idx     [B, Q, K]     int32 selected entries (distinct; -1 = empty slot)
 *   kv_raw  [B, R, D]     prepared raw-token rows for the window
 *   raw_pos0 [B]          int32 position of kv_raw row 0
 *   q_pos   [B, Q]        int32 query positions (negative -> 0)
 *   sinks   [H]           float32 sink logits (-inf allowed)
 *   out     [B, Q, H, D]  out_dtype CAKV_BF16 or CAKV_F32
 *   lse     [B, Q, H]     float32 log-sum-exp (natural log) incl. the sink, or NULL
 * A query with no keys and a -inf sink gets a zero output and lse = -inf.
 * Supported: D in {64, 128, 256, 512}, 1 <= H <= 128, K <= 65536.
 * Workspace: cakv_sparse_mqa_workspace(...) bytes, 256-byte aligned.  It holds
 * the partials of the key-range splits; 0 (workspace may be NULL) when every
 * query runs as a single split, whose kernel writes the output directly.
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE.
 * ------------------------------------------------------------------------- */
size_t cakv_sparse_mqa_workspace(int64_t B, int64_t Q, int32_t H, int32_t D, int32_t K,
                                 int32_t n_win);
int cakv_sparse_mqa_fwd(const cakv_attn_params* p, const void* q, const void* kv_c,
                        const int32_t* idx, const void* kv_raw, const int32_t* raw_pos0,
                        const int32_t* q_pos, const float* sinks, int act_dtype, int64_t B,
                        int64_t Q, int32_t H, int32_t D, int64_t N, int32_t K, int64_t R,
                        void* out, int out_dtype, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * dense_compressed_mqa_fwd  [V4 digest, HCA paragraph: dense attention over
 * all compressed blocks, no sparse selection; V4-Pro card: HCA m'=128]
 *
 * As sparse_mqa_fwd with every visible entry j < min(floor(t/m), N) in place
 * of the idx list.  With m = 4 and an idx list holding every visible entry
 * the two calls compute the same function.
 * Workspace: cakv_dense_mqa_workspace(B, Q, H, D, N, n_win) bytes.
 * ------------------------------------------------------------------------- */
size_t cakv_dense_mqa_workspace(int64_t B, int64_t Q, int32_t H, int32_t D, int64_t N,
                                int32_t n_win);
int cakv_dense_compressed_mqa_fwd(const cakv_attn_params* p, const void* q, const void* kv_c,
                                  const void* kv_raw, const int32_t* raw_pos0,
                                  const int32_t* q_pos, const float* sinks, int act_dtype,
                                  int64_t B, int64_t Q, int32_t H, int32_t D, int64_t N,
                                  int64_t R, void* out, int out_dtype, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CAKV_H */
