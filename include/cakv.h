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
 *   D        4 .. 4096, a multiple of 4
 * Errors: EINVAL (NULL pointers, sizes, dtypes), EUNSUPPORTED (m, D).
 * ------------------------------------------------------------------------- */
int cakv_kv_compress(const void* x, int x_dtype, const float* gate, int64_t B, int64_t T,
                     int64_t D, int32_t m, void* out, int out_dtype, float* out_scale,
                     void* stream);

/* ---------------------------------------------------------------------------
 * kv_compress_ex  [V4 digest, HCA paragraph: HCA's compression is stated to
 * be non-overlapping, which leaves CSA's free to overlap; CSA step 1: the
 * merge uses learned, attention-like weights; Visualised, Dual Compression
 * and Indexing: learned weighted averages]
 *
 * The compressor's variants.  Entry j covers the span
 *     S_j = [max(0, (j+1)*m - span), (j+1)*m)
 * of tokens ending where block j ends (span >= m; span = m is kv_compress),
 * so entries keep the visibility rule of the other calls (entry j is visible
 * at t >= (j+1)*m).  With gate_per_channel = 0 the gate is [B, T], one logit
 * per token; with 1 it is [B, T, D] and every channel d has its own softmax:
 *     a_{i,d} = softmax_{i in S_j}(gate[b, i, d]);  out[b, j, d] = sum_{i in S_j} a_{i,d} x[b, i, d]
 * Entries exist for j < floor(T/m).  Other arguments, dtypes, the fp8 scale
 * rule, sizes and errors as kv_compress; m <= span <= 8192.
 * ------------------------------------------------------------------------- */
int cakv_kv_compress_ex(const void* x, int x_dtype, const float* gate, int gate_per_channel, int64_t B,
                        int64_t T, int64_t D, int32_t m, int32_t span, void* out, int out_dtype,
                        float* out_scale, void* stream);

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
 * Arithmetic in fp32.  Range: the attention calls keep their key-split
 * partials (a convex combination of prepared rows) in fp16, so every
 * prepared element must stay below 65,504 in magnitude; a normalised row
 * has no element above sqrt(D), so this holds whenever every |gamma_kv|
 * is at most 65504 / sqrt(D) (2,896 at D = 512).
 * Errors: EINVAL (NULL pointers, alignment, ranges, positions beyond int32),
 * EUNSUPPORTED (D).
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
 * Inputs must be finite.  Supported sizes: fp32 mode HI 1 .. 64, dI a
 * multiple of 4, HI * dI <= 8192; bf16 mode HI in {32, 64} and dI in
 * {64, 128}; k 1 .. 4096; N < 2^31.
 * Workspace: at least cakv_indexer_topk_workspace(B, Q, N, k) bytes, 256-byte
 * aligned; its contents on entry do not matter.  The size depends only on
 * B, Q and N: both modes share the top-k stage, whose buffers (one 4-byte
 * score key per entry, per-query histograms and candidate lists) do not
 * depend on the key or query dtype, and with Q > 1 it also holds a copy of
 * the keys repacked for the score kernel (B * ceil(N/32) * 4 KiB, sized for
 * dI = 128), so the query takes no dtype argument.
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE.
 * ------------------------------------------------------------------------- */
size_t cakv_indexer_topk_workspace(int64_t B, int64_t Q, int64_t N, int32_t k);
int cakv_indexer_topk(const void* q_idx, int q_dtype, const float* w, const void* k_idx,
                      int k_dtype, const float* k_scale, const int32_t* q_pos, int64_t B,
                      int64_t Q, int64_t N, int32_t HI, int32_t dI, int32_t m, int32_t k,
                      int32_t* idx, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * indexer_topk_noalloc -- for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.
 *
 * cakv_indexer_topk with the same arguments, results and kernels, minus the
 * workspace: the library keeps it in a static device array of
 * CAKV_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held until the process ends.
 * Nothing is allocated; the first call on each device looks up the array's
 * device address with that device current.  Calls whose
 * cakv_indexer_topk_workspace(B, Q, N, k) exceeds the array return
 * CAKV_EWORKSPACE (for example B*Q = 8 queries over N = 262,144 entries need
 * about 9 MB; up to 58 one-query sequences over 262,144 entries fit).  Every call
 * on one GPU shares that GPU's array, and each call clears what it needs
 * cleared itself: calls that can overlap on one GPU (two streams, two
 * threads) race and must be serialised by the caller.
 * Errors: as cakv_indexer_topk; EWORKSPACE (too large), ELAUNCH (the device
 * address could not be looked up).
 * ------------------------------------------------------------------------- */
#define CAKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int cakv_indexer_topk_noalloc(const void* q_idx, int q_dtype, const float* w, const void* k_idx,
                              int k_dtype, const float* k_scale, const int32_t* q_pos, int64_t B,
                              int64_t Q, int64_t N, int32_t HI, int32_t dI, int32_t m, int32_t k,
                              int32_t* idx, void* stream);

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
    int32_t raw_ring;         /* 0: kv_raw row r of sequence b holds position
                                 raw_pos0[b] + r.  1: kv_raw is a ring of R rows,
                                 row p mod R holding position p, kept by
                                 cakv_kv_append (raw_pos0 is not read and may
                                 be NULL); requires R >= n_win, and the ring
                                 must hold the window of every query (its
                                 last n_win positions up to t) */
} cakv_attn_params;

/* ---------------------------------------------------------------------------
 * kv_append  [V4-Pro card, Hybrid attention: a window of the n_win most recent
 * uncompressed tokens on every CSA/HCA layer, because compressed keys cannot
 * reach inside the block being filled; V4 digest, CSA step 1 and HCA
 * paragraph: every m tokens become one entry once the block is complete]
 *
 * The streaming side of a decode step: one new token per sequence enters one
 * compressor's state.  For sequence b with the new token at t = pos[b]
 * (t < 0: nothing for this sequence):
 *   1. raw_ring[b, t mod Rr] = x_tok[b]; gate_ring[b, t mod Rr] = gate_tok[b];
 *   2. if win_ring: win_ring[b, t mod Rw] = the token prepared at position t
 *      (as cakv_kv_prepare computes it: RMSNorm with gamma_kv, RoPE);
 *   3. if (t + 1) mod m == 0 and j = (t + 1)/m - 1 < N: entry j is compressed
 *      as cakv_kv_compress_ex computes it from the tokens of its span
 *      [max(0, t + 1 - span), t] (the earlier ones read from the raw ring) and
 *      stored in cache[b, j]: prepared at position j*m + entry_pos_offset when
 *      prep is given, else as is (fp8 caches: codes and cache_scale[b, j]).
 * Streaming a sequence token by token this way leaves bitwise the cache and
 * the prepared rows that the bulk calls (kv_compress_ex, kv_prepare) write.
 *   x_tok     [B, D]      act_dtype CAKV_F32 or CAKV_BF16
 *   gate_tok  [B] float32, or [B, D] with gate_per_channel = 1
 *   pos       [B] int32
 *   raw_ring  [B, Rr, D]  act_dtype; Rr >= span.  It must already hold the
 *             span's earlier tokens (earlier appends leave them there)
 *   gate_ring [B, Rr] float32, or [B, Rr, D]
 *   win_ring  [B, Rw, D]  act_dtype prepared rows (prep required), or NULL;
 *             the attention calls read it as kv_raw with raw_ring = 1
 *   cache     [B, N, D]  cache_dtype = act_dtype (entries prepared when prep
 *             is given, stored as compressed otherwise) or CAKV_FP8_E4M3
 *             with cache_scale [B, N] float32 (prep NULL)
 *   prep      RMSNorm/RoPE parameters of the cache entries and window rows,
 *             or NULL for a cache of unprepared entries (indexer keys)
 *   D 8 .. 4096 a multiple of 8; m 1 .. 4096; m <= span <= 8192.
 * A decode step of a CSA layer is four calls on one stream: kv_append of the
 * token's KV (cache kv_c, window ring), kv_append of its indexer key (fp8
 * cache, no window), indexer_topk, sparse_mqa_fwd with raw_ring = 1; an HCA
 * layer's is kv_append (m = 128) and dense_compressed_mqa_fwd.  Every call
 * is asynchronous, allocates nothing and has a fixed launch shape, so a step
 * can be captured in a HIP graph.
 * Errors: EINVAL (pointers, dtypes, ring sizes, positions beyond int32),
 * EUNSUPPORTED (D, m, span).
 * ------------------------------------------------------------------------- */
typedef struct cakv_prep_params {
    int32_t rope_dims;        /* r: rotated trailing dims, even, 0 .. D */
    float rope_base;
    int32_t entry_pos_offset; /* entry j sits at position j*m + entry_pos_offset */
    float rms_eps;
    const float* gamma_kv;    /* [D] device pointer, NULL = all ones */
} cakv_prep_params;

int cakv_kv_append(const void* x_tok, const float* gate_tok, int gate_per_channel, const int32_t* pos,
                   int act_dtype, int64_t B, int64_t D, void* raw_ring, float* gate_ring, int64_t Rr,
                   void* win_ring, int64_t Rw, void* cache, int cache_dtype, float* cache_scale, int64_t N,
                   int32_t m, int32_t span, const cakv_prep_params* prep, void* stream);

/* ---------------------------------------------------------------------------
 * kv_append_batch  [the same passages as kv_append]
 *
 * Up to CAKV_APPEND_BATCH_MAX appends of the same B new tokens (positions
 * pos [B] int32, shared) in one launch, for example the three compressors a
 * decode step feeds (a CSA layer's KV and indexer key, an HCA layer's KV):
 * append i does exactly what cakv_kv_append does with the fields of
 * calls[i] (same meaning, layouts and limits as its arguments), so the
 * results are bitwise those of n separate calls.  The appends run
 * concurrently: no two may write the same buffer (their raw rings, gate
 * rings, window rings, caches and scales are distinct; calls whose pointers
 * coincide are refused).  calls is a host array of n descriptors, read
 * before the call returns.
 * Errors: EINVAL (calls NULL, n outside 1 .. CAKV_APPEND_BATCH_MAX, two
 * appends writing the same buffer), and every error of cakv_kv_append for
 * any of the descriptors (nothing is launched then).
 * ------------------------------------------------------------------------- */
#define CAKV_APPEND_BATCH_MAX 4

typedef struct cakv_append_call {
    const void* x_tok;     /* [B, D] act_dtype */
    const float* gate_tok; /* [B] or [B, D] */
    int32_t gate_per_channel;
    int32_t act_dtype;
    int64_t D;
    void* raw_ring;        /* [B, Rr, D] */
    float* gate_ring;      /* [B, Rr] or [B, Rr, D] */
    int64_t Rr;
    void* win_ring;        /* [B, Rw, D] prepared rows, or NULL */
    int64_t Rw;
    void* cache;           /* [B, N, D] */
    int32_t cache_dtype;
    int32_t m;
    float* cache_scale;    /* [B, N], fp8 caches only */
    int64_t N;
    int32_t span;
    const cakv_prep_params* prep;
} cakv_append_call;

int cakv_kv_append_batch(const cakv_append_call* calls, int32_t n, const int32_t* pos, int64_t B, void* stream);

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
 * Supported: D in {128, 512} for CAKV_BF16 activations and D = 128 for
 * CAKV_F32 activations, 1 <= H <= 128, 0 <= K <= 65536, m 1 .. 4096,
 * n_win 0 .. 4096, rope_dims even and at most 64.
 * Workspace: cakv_sparse_mqa_workspace(...) bytes, 256-byte aligned.  It holds
 * the partials of the key-range splits; 0 (workspace may be NULL) when every
 * query runs as a single split, whose kernel writes the output directly.  The
 * reported size never decreases as B*Q grows: a workspace sized for the
 * largest batch serves every smaller batch of the same H, D, K and n_win.
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

/* ===========================================================================
 * Backward pass (training)  [V4-Pro card, section 5 "1M context, gradually":
 * sparse attention is trained from 64K context on, after a short warm-up of
 * the Lightning Indexer].  The gradients of the calls above.  Buffers named
 * "accumulated" receive += (the caller zeroes them); all others are
 * overwritten.  Where float atomics add the contributions of different
 * workgroups (stated per call), results may differ in the last bits run to
 * run.
 * ======================================================================== */

/* ---------------------------------------------------------------------------
 * mqa_bwd: gradient of sparse_mqa_fwd (idx given) or dense_compressed_mqa_fwd
 * (idx NULL), from the forward's inputs, its output `out` and `lse`, and
 * dout [B,Q,H,D] float32.  Per query and head, with do = RoPE_t(dout) (the
 * transpose of the output's rotation by -t), P the softmax weights
 * exp(logit - lse), o = RoPE_t(out) and delta = do . o:
 *     dl_u = P_u (do . k_u - delta),   dsink = -P_sink delta,
 *     dq_hat = tau sum_u dl_u k_u,     dk_u += tau dl_u q_hat + P_u do,
 * then dq through RoPE_t's transpose and the RMSNorm (with gamma_q) of q.
 *   dq       [B,Q,H,D] float32, overwritten (gradient of the raw query)
 *   dkv_c    [B,N,D]   float32, accumulated: gradient of the prepared cache
 *            rows (what the forward reads; cakv_kv_prepare_bwd continues to
 *            the raw entries)
 *   dkv_raw  [B,R,D]   float32, accumulated: the same for the window rows
 *   dsinks   [H] float32 accumulated, or NULL; dgamma_q [D] accumulated or NULL
 * Supported: CAKV_BF16 activations with D = 512, 1 <= H <= 128,
 * B*Q <= 65535; other parameters as the forward (ring mode included).
 * The selected entries of a query must be distinct (as for the forward):
 * with Q = 1 every key row is then touched by one workgroup only, and its
 * gradient is added without atomics (bitwise deterministic); with Q > 1
 * rows shared by a sequence's queries are added with float atomics.
 * Workspace: cakv_mqa_bwd_workspace(B, Q, H, D, n_keys, n_win) bytes with
 * n_keys = K (sparse) or N (dense), 256-byte aligned.
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE.
 * ------------------------------------------------------------------------- */
size_t cakv_mqa_bwd_workspace(int64_t B, int64_t Q, int32_t H, int32_t D, int64_t n_keys, int32_t n_win);
int cakv_mqa_bwd(const cakv_attn_params* p, const void* q, const void* kv_c, const int32_t* idx,
                 const void* kv_raw, const int32_t* raw_pos0, const int32_t* q_pos, const float* sinks,
                 int act_dtype, int64_t B, int64_t Q, int32_t H, int32_t D, int64_t N, int32_t K, int64_t R,
                 const void* out, int out_dtype, const float* lse, const float* dout, float* dq,
                 float* dkv_c, float* dkv_raw, float* dsinks, float* dgamma_q, void* workspace,
                 size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kv_prepare_bwd: gradient of cakv_kv_prepare for entries j0 .. j0+n-1:
 * dy [B,N,D] float32 (gradient of the prepared rows) -> dx [B,N,D] float32
 * (gradient of the raw entries kv_in, rows j0 .. j0+n-1 overwritten, the
 * others untouched); dgamma_kv [D] accumulated, or NULL.  The rotation's
 * transpose is the rotation by -position; then the RMSNorm gradient
 *     dx = gamma du / r - x sum_d(gamma_d du_d x_d) / (D r^3).
 * Arguments and limits otherwise as cakv_kv_prepare.
 * ------------------------------------------------------------------------- */
int cakv_kv_prepare_bwd(const void* kv_in, int act_dtype, const float* dy, float* dx, float* dgamma_kv,
                        int64_t B, int64_t N, int64_t D, int64_t j0, int64_t n, const float* gamma_kv,
                        int32_t m, int32_t rope_dims, float rope_base, int32_t entry_pos_offset,
                        float rms_eps, void* stream);

/* ---------------------------------------------------------------------------
 * kv_compress_bwd: gradient of cakv_kv_compress_ex (and cakv_kv_compress:
 * span = m, per-token gates).  dc [B, floor(T/m), D] float32 ->
 *     dx[b,i,d] = sum_{j: i in S_j} a_{i,d} dc[b,j,d]
 *     dgate[b,i(,d)] = sum_{j: i in S_j} (sum_d) a_{i,d} (x[b,i,d] - c[b,j,d]) dc[b,j,d]
 * dx [B,T,D] float32 and dgate ([B,T] or [B,T,D] float32) overwritten
 * (tokens in no entry's span get 0).  Workspace
 * cakv_kv_compress_bwd_workspace(B, T, D, m) bytes (the entries' softmax
 * statistics).  Arguments and limits otherwise as cakv_kv_compress_ex.
 * ------------------------------------------------------------------------- */
size_t cakv_kv_compress_bwd_workspace(int64_t B, int64_t T, int64_t D, int32_t m);
int cakv_kv_compress_bwd(const void* x, int x_dtype, const float* gate, int gate_per_channel, int64_t B,
                         int64_t T, int64_t D, int32_t m, int32_t span, const float* dc, float* dx,
                         float* dgate, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * indexer_bwd: gradient of the indexer score S(j) = sum_h w_h ReLU(q_h . k_j)
 * over the selected entries idx [B,Q,K] (slots that are -1 or not visible
 * carry nothing), given dS [B,Q,K] float32:
 *     dq_h += dS_j w_h [s_h > 0] k_j,  dw_h += dS_j ReLU(s_h),
 *     dk_j += dS_j sum_h w_h [s_h > 0] q_h.
 * Each ReLU decision is taken on the forward's canonical fp32 dot product
 * (head dim ascending from +0 in fmaf, fp8 keys decoded exactly), whatever
 * the mode.  dq_idx [B,Q,HI,dI] and dw [B,Q,HI] float32 overwritten; dk
 * [B,N,dI] float32 accumulated.  Modes and dtypes as cakv_indexer_topk;
 * HI <= 64, dI a multiple of 8 up to 128, K <= 65536, B*Q < 2^23.
 * ------------------------------------------------------------------------- */
int cakv_indexer_bwd(const void* q_idx, int q_dtype, const float* w, const void* k_idx, int k_dtype,
                     const float* k_scale, const int32_t* q_pos, const int32_t* idx, const float* dS, int64_t B,
                     int64_t Q, int64_t N, int32_t HI, int32_t dI, int32_t m, int32_t K, float* dq_idx,
                     float* dw, float* dk, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CAKV_H */
