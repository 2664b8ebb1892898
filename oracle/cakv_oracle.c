/*
 * cakv_oracle.c -- plain, slow CPU reference of the compressed-attention hot
 * path (DeepSeek-V4 CSA / HCA attention).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the HIP library, and the HIP library never calls it.
 *
 * Sources (the pages this follows; cited by short name below):
 *   [V4-Pro card]   "DeepSeek V4-Pro", llm-arch-kb (lizeman.github.io),
 *                   section "What's new in V4", item 1 "Hybrid attention".
 *   [V4 digest]     DeepSeek V4 technical-report digest (agentupdate.ai, in
 *                   Chinese), section on hybrid attention: the four CSA steps
 *                   and the HCA paragraph.
 *   [Visualised]    "DeepSeek V4-Pro Architecture: KV Cache Compression and
 *                   Hyper-Connections Visualised" (webconsulting.at),
 *                   "Key points" and "Dual Compression and Indexing".
 *
 * Readings where the pages leave a step open (each one is a parameter or a
 * stated rule, shared with the GPU path only through its documented meaning):
 *   - compressor weights: softmax over one gate logit per raw token inside
 *     each block of m tokens; blocks do not overlap;
 *   - indexer score: sum over indexer heads h of w_h * ReLU(q_h . k), one key
 *     per compressed entry shared by all indexer heads, no scale;
 *   - top-k order: score descending, ties to the lower index; output sorted
 *     ascending by index and padded with -1;
 *   - visibility: compressed entry j is visible to a query at position t iff
 *     its whole block precedes t, i.e. j < floor(t/m) (and j < N);
 *   - window: raw positions max(0, t-n_win+1) .. t, the query's own token
 *     included; one joint softmax over compressed keys, window keys and the
 *     sink (whose value is zero);
 *   - K = V = the RMS-normalised, rotated KV vector; rotation on the last r
 *     dims in consecutive pairs with angle pos * base^(-2i/r); compressed
 *     entry j sits at position j*m + entry_pos_offset; the output is rotated
 *     back by -t.
 *
 * Precision: the indexer score is computed in fp32 with explicit fmaf chains
 * in a fixed order (head-dim ascending, then heads ascending), because the
 * fp32 indexer mode of the library must reproduce it bit for bit.  All other
 * steps compute in fp64 and return fp64.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef int64_t i64;

#define OR_F32 0
#define OR_BF16 1

#define OR_OK 0
#define OR_EINVAL (-1)

static float bf16_bits_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* exact value of element i of a float32 or bf16 (raw bits) array */
static double load_elem(const void* p, int dtype, i64 i) {
    if (dtype == OR_F32) return (double)((const float*)p)[i];
    return (double)bf16_bits_to_float(((const uint16_t*)p)[i]);
}

static float load_elem_f(const void* p, int dtype, i64 i) {
    if (dtype == OR_F32) return ((const float*)p)[i];
    return bf16_bits_to_float(((const uint16_t*)p)[i]);
}

/* ------------------------------------------------------------------------ */
/* O1  KV compression [V4 digest, CSA step 1; HCA paragraph] [V4-Pro card]   */
/*     c_j = sum_i softmax(g[jm .. jm+m-1])_i * x[jm+i], blocks of m tokens.  */
/*     Only whole blocks are produced.                                       */
/* ------------------------------------------------------------------------ */
int oracle_kv_compress(const void* x, int x_dtype, const float* g, i64 B, i64 T, i64 D,
                       int m, double* out) {
    if (m < 1 || B < 0 || T < 0 || D < 1) return OR_EINVAL;
    i64 nb = T / m;
#pragma omp parallel for schedule(static)
    for (i64 bj = 0; bj < B * nb; ++bj) {
        i64 b = bj / nb, j = bj % nb;
        double* a = (double*)malloc(sizeof(double) * (size_t)m);
        {
            const float* gb = g + b * T + j * m;
            double mx = -INFINITY;
            for (int i = 0; i < m; ++i)
                if ((double)gb[i] > mx) mx = (double)gb[i];
            double z = 0.0;
            for (int i = 0; i < m; ++i) {
                a[i] = exp((double)gb[i] - mx);
                z += a[i];
            }
            for (int i = 0; i < m; ++i) a[i] /= z;
            double* o = out + (b * nb + j) * D;
            for (i64 d = 0; d < D; ++d) {
                double s = 0.0;
                for (int i = 0; i < m; ++i)
                    s += a[i] * load_elem(x, x_dtype, (b * T + j * m + i) * D + d);
                o[d] = s;
            }
        }
        free(a);
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* O1x compression variants [V4 digest, HCA paragraph: the HCA compressor is */
/*     stated to be non-overlapping, which leaves room for CSA blocks that   */
/*     overlap; CSA step 1: the block is merged by learned, attention-like   */
/*     weights] [Visualised, Dual Compression and Indexing: learned weighted */
/*     averages].                                                            */
/*     Readings: entry j still ends where block j ends, so its visibility is */
/*     unchanged; it covers the `span` tokens before that end (span >= m;    */
/*     span = m is the plain compressor), cut at token 0.  The gate is one   */
/*     logit per token, or one per token and channel (then every channel has */
/*     its own softmax over the entry's tokens):                             */
/*       S_j = [max(0, (j+1)m - span), (j+1)m),                              */
/*       a_{i,d} = exp(g_{i,d}) / sum_{i' in S_j} exp(g_{i',d}),             */
/*       c_j[d]  = sum_{i in S_j} a_{i,d} x_i[d].                            */
/*     Entries exist for the whole strides j < floor(T/m).                   */
/* ------------------------------------------------------------------------ */
int oracle_kv_compress_ex(const void* x, int x_dtype, const float* g, int gate_per_channel, i64 B, i64 T,
                          i64 D, int m, int span, double* out) {
    if (m < 1 || span < m || B < 0 || T < 0 || D < 1) return OR_EINVAL;
    i64 nb = T / m;
#pragma omp parallel for schedule(static)
    for (i64 bj = 0; bj < B * nb; ++bj) {
        i64 b = bj / nb, j = bj % nb;
        i64 hi = (j + 1) * m, lo = hi - span < 0 ? 0 : hi - span;
        i64 n = hi - lo;
        double* a = (double*)malloc(sizeof(double) * (size_t)n);
        double* o = out + (b * nb + j) * D;
        for (i64 d = 0; d < D; ++d) {
            /* the softmax of this channel's logits over the entry's tokens */
            if (d == 0 || gate_per_channel) {
                double mx = -INFINITY, z = 0.0;
                for (i64 i = 0; i < n; ++i) {
                    double gi = gate_per_channel ? (double)g[(b * T + lo + i) * D + d] : (double)g[b * T + lo + i];
                    if (gi > mx) mx = gi;
                }
                for (i64 i = 0; i < n; ++i) {
                    double gi = gate_per_channel ? (double)g[(b * T + lo + i) * D + d] : (double)g[b * T + lo + i];
                    a[i] = exp(gi - mx);
                    z += a[i];
                }
                for (i64 i = 0; i < n; ++i) a[i] /= z;
            }
            double s = 0.0;
            for (i64 i = 0; i < n; ++i) s += a[i] * load_elem(x, x_dtype, (b * T + lo + i) * D + d);
            o[d] = s;
        }
        free(a);
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* fp8 E4M3 (OCP "E4M3FN"): 1 sign bit, 4 exponent bits with bias 7, 3       */
/* mantissa bits; exponent field 0 holds subnormals M * 2^-9; no infinities;  */
/* S.1111.111 is NaN; largest finite magnitude 448.                          */
/* The "low precision" cheap similarity pass of [Visualised, Dual            */
/* Compression and Indexing] is read as fp8 indexer keys with one            */
/* power-of-two scale per compressed entry.                                  */
/* ------------------------------------------------------------------------ */
double oracle_e4m3_decode(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, mt = code & 7;
    double v;
    if (e == 15 && mt == 7) return NAN;
    if (e == 0) v = ldexp((double)mt, -9);
    else v = ldexp(1.0 + mt / 8.0, e - 7);
    return s ? -v : v;
}

/* Round-to-nearest-even to E4M3, saturating at +-448.  The 127 finite
 * non-negative codes 0x00..0x7E have strictly increasing magnitudes, so the
 * nearest code is found by bisection over their decoded values; an exact tie
 * between two neighbours goes to the code whose lowest mantissa bit is 0. */
int oracle_e4m3_encode(double v) {
    static double mag[127];
    static int ready = 0;
    if (!ready) { /* benign: every thread writes the same values */
        for (int c = 0; c <= 0x7E; ++c) mag[c] = oracle_e4m3_decode(c);
        ready = 1;
    }
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v);
    int best;
    if (a >= 448.0) {
        best = 0x7E;
    } else {
        int lo = 0, hi = 0x7E; /* invariant: mag[lo] <= a < mag[hi] */
        while (hi - lo > 1) {
            int mid = (lo + hi) / 2;
            if (mag[mid] <= a) lo = mid;
            else hi = mid;
        }
        double dlo = a - mag[lo], dhi = mag[hi] - a;
        if (dlo < dhi) best = lo;
        else if (dhi < dlo) best = hi;
        else best = (lo & 1) == 0 ? lo : hi;
    }
    return best | (neg << 7);
}

/* Q8: per-entry power-of-two scale s = 2^e, e the smallest integer >= -126
 * with max_d |c_d| <= 448 * 2^e (e = 0 for an all-zero row); codes are
 * E4M3(c_d / s).  The dequantised key is code * s, exact in fp32. */
int oracle_q8_quantize(const void* c, int c_is_f64, i64 n, i64 D, uint8_t* code, float* scale) {
    int bad = 0;
    (void)oracle_e4m3_encode(0.0); /* fill the magnitude table before the threads start */
#pragma omp parallel for schedule(static)
    for (i64 j = 0; j < n; ++j) {
        double A = 0.0;
        for (i64 d = 0; d < D; ++d) {
            double x = c_is_f64 ? ((const double*)c)[j * D + d] : (double)((const float*)c)[j * D + d];
            if (!isfinite(x)) {
#pragma omp atomic write
                bad = 1;
            }
            if (fabs(x) > A) A = fabs(x);
        }
        int e = 0;
        if (A > 0.0 && isfinite(A)) {
            e = -126;
            while (A > ldexp(448.0, e)) ++e;
        }
        scale[j] = (float)ldexp(1.0, e);
        for (i64 d = 0; d < D; ++d) {
            double x = c_is_f64 ? ((const double*)c)[j * D + d] : (double)((const float*)c)[j * D + d];
            code[j * D + d] = (uint8_t)oracle_e4m3_encode(ldexp(x, -e));
        }
    }
    return bad ? OR_EINVAL : OR_OK;
}

/* ------------------------------------------------------------------------ */
/* O2  Lightning-indexer score [V4 digest, CSA step 2] [V4-Pro card]         */
/*     S(t, j) = sum_h w[t,h] * ReLU(q_I[t,h,:] . k_I[j,:]) for j < n_vis(t). */
/*     Canonical fp32 order: for each head an fmaf chain over d ascending    */
/*     from +0, ReLU as (s > 0 ? s : +0), then an fmaf chain over h           */
/*     ascending from +0.                                                    */
/* ------------------------------------------------------------------------ */
static i64 n_visible(i64 t, int m, i64 N) {
    i64 nv = t / m;
    return nv < N ? nv : N;
}

/* key input: either float32 keys (k_code == NULL) or fp8 codes with one
 * scale per entry, dequantised exactly as code * scale. */
static void key_row(const float* kf, const uint8_t* kc, const float* ks, i64 row, i64 dI, float* dst) {
    for (i64 d = 0; d < dI; ++d)
        dst[d] = kc ? (float)oracle_e4m3_decode(kc[row * dI + d]) * ks[row] : kf[row * dI + d];
}

/* rows: flattened (b*Q + q) query rows to score, or NULL for all; scores is
 * [n_rows][N] with NaN at invisible entries; n_vis is [n_rows]. */
int oracle_indexer_scores(const void* q_idx, int q_dtype, const float* w, const float* k_f32,
                          const uint8_t* k_code, const float* k_scale, const int32_t* q_pos,
                          i64 B, i64 Q, i64 N, int HI, int dI, int m, const i64* rows,
                          i64 n_rows, float* scores, int32_t* n_vis) {
    if (m < 1 || HI < 1 || dI < 1) return OR_EINVAL;
    if (!rows) n_rows = B * Q;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (i64 r = 0; r < n_rows; ++r) {
        i64 bq = rows ? rows[r] : r;
        if (bq < 0 || bq >= B * Q || q_pos[bq] < 0) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        i64 b = bq / Q;
        i64 t = q_pos[bq];
        i64 nv = n_visible(t, m, N);
        n_vis[r] = (int32_t)nv;
        float* out = scores + r * N;
        float* qf = (float*)malloc(sizeof(float) * (size_t)HI * dI);
        float* kr = (float*)malloc(sizeof(float) * (size_t)dI);
        for (i64 i = 0; i < (i64)HI * dI; ++i) qf[i] = load_elem_f(q_idx, q_dtype, bq * HI * dI + i);
        const float* wr = w + bq * HI;
        for (i64 j = 0; j < N; ++j) {
            if (j >= nv) {
                out[j] = NAN;
                continue;
            }
            key_row(k_f32, k_code, k_scale, b * N + j, dI, kr);
            float S = 0.0f;
            for (int h = 0; h < HI; ++h) {
                float s = 0.0f;
                for (int d = 0; d < dI; ++d)
                    s = fmaf(qf[h * dI + d], kr[d], s);
                float rl = (s > 0.0f) ? s : 0.0f;
                S = fmaf(wr[h], rl, S);
            }
            out[j] = S;
        }
        free(qf);
        free(kr);
    }
    return bad ? OR_EINVAL : OR_OK;
}

/* ------------------------------------------------------------------------ */
/* O3  top-k [V4 digest, CSA step 2 and the two-level reduction remark]      */
/*     [Visualised, Key points: ~262,000 entries -> top 1,024]               */
/*     Strict order: higher score first, equal scores by lower index.        */
/*     Keep the first min(k, n_vis), sort them by index, pad with -1.        */
/* ------------------------------------------------------------------------ */
typedef struct {
    float s;
    int32_t j;
} scored_t;

static int cmp_rank(const void* a, const void* b) {
    const scored_t* x = (const scored_t*)a;
    const scored_t* y = (const scored_t*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int cmp_i32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

int oracle_topk(const float* scores, const int32_t* n_vis, i64 n_rows, i64 N, int k, int32_t* idx) {
    if (k < 1) return OR_EINVAL;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (i64 r = 0; r < n_rows; ++r) {
        i64 nv = n_vis[r];
        int32_t* o = idx + r * k;
        if (nv < 0 || nv > N) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        scored_t* v = (scored_t*)malloc(sizeof(scored_t) * (size_t)(nv > 0 ? nv : 1));
        for (i64 j = 0; j < nv; ++j) {
            float s = scores[r * N + j];
            if (isnan(s)) {
#pragma omp atomic write
                bad = 1;
            }
            v[j].s = s;
            v[j].j = (int32_t)j;
        }
        qsort(v, (size_t)nv, sizeof(scored_t), cmp_rank);
        i64 keep = nv < k ? nv : k;
        for (i64 i = 0; i < keep; ++i) o[i] = v[i].j;
        qsort(o, (size_t)keep, sizeof(int32_t), cmp_i32);
        for (i64 i = keep; i < k; ++i) o[i] = -1;
        free(v);
    }
    return bad ? OR_EINVAL : OR_OK;
}

/* ------------------------------------------------------------------------ */
/* O4  core attention [V4-Pro card, Hybrid attention: shared-KV MQA, sliding */
/*     window branch, attention sink, partial RoPE and its inverse on the     */
/*     output, QK RMSNorm] [V4 digest, CSA step 3; HCA paragraph]            */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t m;                /* compression ratio of kv_c */
    int32_t n_win;            /* raw window length */
    int32_t rope_dims;        /* r: rotated trailing dims (even) */
    int32_t entry_pos_offset; /* position of compressed entry j is j*m + this */
    double rope_base;
    double softmax_scale;     /* 0 -> 1/sqrt(D) */
    double rms_eps;
} oracle_attn_params;

static void rms_normalise(const double* x, const float* gamma, i64 D, double eps, double* y) {
    double ss = 0.0;
    for (i64 d = 0; d < D; ++d) ss += x[d] * x[d];
    double inv = 1.0 / sqrt(ss / (double)D + eps);
    for (i64 d = 0; d < D; ++d) y[d] = x[d] * inv * (gamma ? (double)gamma[d] : 1.0);
}

/* rotate the trailing r dims of x (length D) by position pos */
static void rope(double* x, i64 D, int r, double base, double pos) {
    for (int i = 0; i < r / 2; ++i) {
        double theta = pow(base, -2.0 * i / (double)r);
        double ang = pos * theta;
        double c = cos(ang), s = sin(ang);
        i64 a = D - r + 2 * i;
        double x0 = x[a], x1 = x[a + 1];
        x[a] = x0 * c - x1 * s;
        x[a + 1] = x0 * s + x1 * c;
    }
}

/* The key (= value) vector of compressed entry j, a function of the entry
 * alone: RMSNorm with gamma_kv, then the trailing r dims rotated by the
 * entry's position j*m + entry_pos_offset.  [V4-Pro card, "Hybrid
 * attention": RMSNorm on the single compressed KV head before the dot
 * product; RoPE on the last 64 dims of each KV entry.]  Entries j0 .. j0+n-1
 * of each of the B sequences (N entries each); out is [B][n][D].  This is the
 * same per-entry computation the attention below applies to compressed rows. */
int oracle_kv_prepare(const void* kv_c, int act_dtype, const float* gamma_kv, i64 B, i64 N, i64 D,
                      i64 j0, i64 n, int m, int rope_dims, double rope_base, int entry_pos_offset,
                      double rms_eps, double* out) {
    if (B < 0 || N < 0 || D < 1 || j0 < 0 || n < 0 || j0 + n > N || m < 1 || rope_dims < 0 ||
        (rope_dims & 1) || rope_dims > D)
        return OR_EINVAL;
    double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
    for (i64 b = 0; b < B; ++b)
        for (i64 i = 0; i < n; ++i) {
            i64 j = j0 + i;
            for (i64 d = 0; d < D; ++d) tmp[d] = load_elem(kv_c, act_dtype, (b * N + j) * D + d);
            double* y = out + (b * n + i) * D;
            rms_normalise(tmp, gamma_kv, D, rms_eps, y);
            rope(y, D, rope_dims, rope_base, (double)(j * m + entry_pos_offset));
        }
    free(tmp);
    return OR_OK;
}

/* idx == NULL: dense over all visible entries (HCA); otherwise the K slots
 * of idx (entries that are -1 or not visible are skipped).
 * rows: flattened (b*Q+q) rows to compute, or NULL for all; out is
 * [n_rows][H][D], lse is [n_rows][H] (natural log). */
int oracle_attention(const oracle_attn_params* p, const void* q, const void* kv_c,
                     const int32_t* idx, int K, const void* kv_raw, const int32_t* raw_pos0,
                     const int32_t* q_pos, const float* sinks, const float* gamma_q,
                     const float* gamma_kv, int act_dtype, i64 B, i64 Q, i64 H, i64 D, i64 N,
                     i64 R, const i64* rows, i64 n_rows, double* out, double* lse) {
    if (p->m < 1 || p->n_win < 0 || p->rope_dims < 0 || (p->rope_dims & 1) || p->rope_dims > D)
        return OR_EINVAL;
    if (!rows) n_rows = B * Q;
    double tau = p->softmax_scale > 0.0 ? p->softmax_scale : 1.0 / sqrt((double)D);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (i64 r = 0; r < n_rows; ++r) {
        i64 bq = rows ? rows[r] : r;
        if (bq < 0 || bq >= B * Q || q_pos[bq] < 0) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        i64 b = bq / Q;
        i64 t = q_pos[bq];
        i64 nv = n_visible(t, p->m, N);
        /* gather the key set U: compressed entries, then the raw window */
        i64 cap = (idx ? K : nv) + p->n_win;
        double* keys = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1) * D);
        double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
        i64 nk = 0;
        i64 ncomp = idx ? K : nv;
        for (i64 i = 0; i < ncomp; ++i) {
            i64 j = idx ? idx[bq * K + i] : i;
            if (j < 0 || j >= nv) continue;
            for (i64 d = 0; d < D; ++d) tmp[d] = load_elem(kv_c, act_dtype, (b * N + j) * D + d);
            rms_normalise(tmp, gamma_kv, D, p->rms_eps, keys + nk * D);
            rope(keys + nk * D, D, p->rope_dims, p->rope_base, (double)(j * p->m + p->entry_pos_offset));
            ++nk;
        }
        i64 p_lo = t - p->n_win + 1;
        if (p_lo < 0) p_lo = 0;
        for (i64 pos = p_lo; pos <= t && p->n_win > 0; ++pos) {
            i64 row = pos - raw_pos0[b];
            if (row < 0 || row >= R) continue;
            for (i64 d = 0; d < D; ++d) tmp[d] = load_elem(kv_raw, act_dtype, (b * R + row) * D + d);
            rms_normalise(tmp, gamma_kv, D, p->rms_eps, keys + nk * D);
            rope(keys + nk * D, D, p->rope_dims, p->rope_base, (double)pos);
            ++nk;
        }
        double* qh = (double*)malloc(sizeof(double) * (size_t)D);
        double* lg = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        for (i64 h = 0; h < H; ++h) {
            for (i64 d = 0; d < D; ++d) tmp[d] = load_elem(q, act_dtype, (bq * H + h) * D + d);
            rms_normalise(tmp, gamma_q, D, p->rms_eps, qh);
            rope(qh, D, p->rope_dims, p->rope_base, (double)t);
            double mx = (double)sinks[h];
            for (i64 u = 0; u < nk; ++u) {
                double s = 0.0;
                for (i64 d = 0; d < D; ++d) s += qh[d] * keys[u * D + d];
                lg[u] = tau * s;
                if (lg[u] > mx) mx = lg[u];
            }
            double* o = out + (r * H + h) * D;
            if (mx == -INFINITY) { /* no keys and a -inf sink: nothing to attend */
                for (i64 d = 0; d < D; ++d) o[d] = 0.0;
                if (lse) lse[r * H + h] = -INFINITY;
                continue;
            }
            double z = exp((double)sinks[h] - mx);
            for (i64 d = 0; d < D; ++d) o[d] = 0.0;
            for (i64 u = 0; u < nk; ++u) {
                double e = exp(lg[u] - mx);
                z += e;
                for (i64 d = 0; d < D; ++d) o[d] += e * keys[u * D + d];
            }
            for (i64 d = 0; d < D; ++d) o[d] /= z;
            rope(o, D, p->rope_dims, p->rope_base, -(double)t);
            if (lse) lse[r * H + h] = mx + log(z);
        }
        free(qh);
        free(lg);
        free(keys);
        free(tmp);
    }
    return bad ? OR_EINVAL : OR_OK;
}

/* ======================================================================== */
/* Backward pass (training)  [V4-Pro card, section 5 "1M context,            */
/* gradually": sparse attention is trained from 64K context on, after a      */
/* short warm-up of the Lightning Indexer].  The gradients of the forward    */
/* steps above, by the chain rule, in fp64.                                   */
/* ======================================================================== */

/* RMSNorm backward for y = gamma * x / r, r = sqrt(mean(x^2) + eps):
 *   dx_e = gamma_e dy_e / r - x_e sum_d(gamma_d dy_d x_d) / (D r^3),
 *   dgamma_d += dy_d x_d / r.  dgamma may be NULL. */
static void rms_normalise_bwd(const double* x, const float* gamma, i64 D, double eps, const double* dy, double* dx,
                              double* dgamma) {
    double ss = 0.0, dot = 0.0;
    for (i64 d = 0; d < D; ++d) ss += x[d] * x[d];
    double r = sqrt(ss / (double)D + eps);
    for (i64 d = 0; d < D; ++d) dot += (gamma ? (double)gamma[d] : 1.0) * dy[d] * x[d];
    for (i64 d = 0; d < D; ++d) {
        double g = gamma ? (double)gamma[d] : 1.0;
        dx[d] = g * dy[d] / r - x[d] * dot / ((double)D * r * r * r);
        if (dgamma) dgamma[d] += dy[d] * x[d] / r;
    }
}

/* Gradient of kv_prepare: entries j0 .. j0+n-1 of each sequence; dy [B][n][D]
 * is the gradient of the prepared rows, dx [B][n][D] receives the raw
 * entries' gradient, dgamma [D] (or NULL) accumulates gamma_kv's.  The
 * rotation's transpose is the rotation by -position. */
int oracle_kv_prepare_bwd(const void* kv_c, int act_dtype, const float* gamma_kv, i64 B, i64 N, i64 D, i64 j0,
                          i64 n, int m, int rope_dims, double rope_base, int entry_pos_offset, double rms_eps,
                          const double* dy, double* dx, double* dgamma) {
    if (B < 0 || N < 0 || D < 1 || j0 < 0 || n < 0 || j0 + n > N || m < 1 || rope_dims < 0 ||
        (rope_dims & 1) || rope_dims > D)
        return OR_EINVAL;
    double* x = (double*)malloc(sizeof(double) * (size_t)D);
    double* du = (double*)malloc(sizeof(double) * (size_t)D);
    if (dgamma)
        for (i64 d = 0; d < D; ++d) dgamma[d] = 0.0;
    for (i64 b = 0; b < B; ++b)
        for (i64 i = 0; i < n; ++i) {
            i64 j = j0 + i;
            for (i64 d = 0; d < D; ++d) {
                x[d] = load_elem(kv_c, act_dtype, (b * N + j) * D + d);
                du[d] = dy[(b * n + i) * D + d];
            }
            rope(du, D, rope_dims, rope_base, -(double)(j * m + entry_pos_offset));
            rms_normalise_bwd(x, gamma_kv, D, rms_eps, du, dx + (b * n + i) * D, dgamma);
        }
    free(x);
    free(du);
    return OR_OK;
}

/* Gradient of the compression variants (and of the plain compressor, span =
 * m, per-token gates): for each entry j with span S_j and channel d,
 *   c_d = sum_i a_{i,d} x_{i,d},   a = softmax over S_j of the gate,
 *   dx_{i,d} += a_{i,d} dc_d,       dg_{i,d} += a_{i,d} (x_{i,d} - c_d) dc_d
 * (per-token gates sum dg over the channels).  dc is [B][T/m][D]; dx
 * [B][T][D] and dg ([B][T] or [B][T][D]) are overwritten; tokens outside
 * every entry's span get zero. */
int oracle_kv_compress_bwd(const void* x, int x_dtype, const float* g, int gate_per_channel, i64 B, i64 T, i64 D,
                           int m, int span, const double* dc, double* dx, double* dg) {
    if (m < 1 || span < m || B < 0 || T < 0 || D < 1) return OR_EINVAL;
    i64 nb = T / m;
    memset(dx, 0, sizeof(double) * (size_t)(B * T * D));
    memset(dg, 0, sizeof(double) * (size_t)(B * T * (gate_per_channel ? D : 1)));
    double* c = (double*)malloc(sizeof(double) * (size_t)D);
    double* a = (double*)malloc(sizeof(double) * (size_t)span * (size_t)D);
    for (i64 b = 0; b < B; ++b)
        for (i64 j = 0; j < nb; ++j) {
            i64 hi = (j + 1) * m, lo = hi - span < 0 ? 0 : hi - span, n = hi - lo;
            for (i64 d = 0; d < D; ++d) {
                double mx = -INFINITY, z = 0.0;
                for (i64 i = 0; i < n; ++i) {
                    double gi = gate_per_channel ? (double)g[(b * T + lo + i) * D + d] : (double)g[b * T + lo + i];
                    if (gi > mx) mx = gi;
                }
                for (i64 i = 0; i < n; ++i) {
                    double gi = gate_per_channel ? (double)g[(b * T + lo + i) * D + d] : (double)g[b * T + lo + i];
                    a[i * D + d] = exp(gi - mx);
                    z += a[i * D + d];
                }
                c[d] = 0.0;
                for (i64 i = 0; i < n; ++i) {
                    a[i * D + d] /= z;
                    c[d] += a[i * D + d] * load_elem(x, x_dtype, (b * T + lo + i) * D + d);
                }
            }
            const double* dcj = dc + (b * nb + j) * D;
            for (i64 i = 0; i < n; ++i)
                for (i64 d = 0; d < D; ++d) {
                    double xi = load_elem(x, x_dtype, (b * T + lo + i) * D + d);
                    dx[(b * T + lo + i) * D + d] += a[i * D + d] * dcj[d];
                    double gg = a[i * D + d] * (xi - c[d]) * dcj[d];
                    if (gate_per_channel) dg[(b * T + lo + i) * D + d] += gg;
                    else dg[b * T + lo + i] += gg;
                }
        }
    free(c);
    free(a);
    return OR_OK;
}

/* Gradient of the indexer score S(j) = sum_h w_h ReLU(q_h . k_j) over the
 * selected entries idx[b,i,:] (slots that are -1 or not visible carry
 * nothing), given dS [B][Q][K]:
 *   dq_h += dS_j w_h [s_h > 0] k_j,   dw_h += dS_j ReLU(s_h),
 *   dk_j += dS_j sum_h w_h [s_h > 0] q_h.
 * Each ReLU decision [s_h > 0] is taken on the forward's canonical fp32 dot
 * product (head dim ascending from +0 in fmaf), so both sides decide on the
 * same fp32 value; ReLU(s_h) itself and the sums are fp64.  absolute = 1 accumulates |term| instead (with
 * the same decisions): the magnitude of each sum, for error bounds.
 * dq [B][Q][HI][dI], dw [B][Q][HI] and dk [B][N][dI] are overwritten. */
int oracle_indexer_bwd(const void* q_idx, int q_dtype, const float* w, const float* k_f32, const uint8_t* k_code,
                       const float* k_scale, const int32_t* q_pos, const int32_t* idx, i64 B, i64 Q, i64 N, int HI,
                       int dI, int m, int K, const float* dS, int absolute, double* dq, double* dw, double* dk) {
    if (B < 0 || Q < 0 || N < 0 || HI < 1 || dI < 1 || m < 1 || K < 0) return OR_EINVAL;
    memset(dq, 0, sizeof(double) * (size_t)(B * Q * HI * dI));
    memset(dw, 0, sizeof(double) * (size_t)(B * Q * HI));
    memset(dk, 0, sizeof(double) * (size_t)(B * N * dI));
    float* kr = (float*)malloc(sizeof(float) * (size_t)dI);
    for (i64 bq = 0; bq < B * Q; ++bq) {
        i64 b = bq / Q;
        if (q_pos[bq] < 0) continue;
        i64 nv = n_visible(q_pos[bq], m, N);
        for (int s = 0; s < K; ++s) {
            i64 j = idx[bq * K + s];
            if (j < 0 || j >= nv) continue;
            key_row(k_f32, k_code, k_scale, b * N + j, dI, kr);
            double g = (double)dS[bq * K + s];
            for (int h = 0; h < HI; ++h) {
                float sh = 0.0f;
                double s64 = 0.0;
                for (int d = 0; d < dI; ++d) {
                    sh = fmaf(load_elem_f(q_idx, q_dtype, (bq * HI + h) * dI + d), kr[d], sh);
                    s64 += load_elem(q_idx, q_dtype, (bq * HI + h) * dI + d) * (double)kr[d];
                }
                double wh = (double)w[bq * HI + h];
                /* the decision on the forward's fp32 score, the value exact */
                double relu = sh > 0.0f ? s64 : 0.0;
                dw[bq * HI + h] += absolute ? fabs(g * relu) : g * relu;
                if (!(sh > 0.0f)) continue;
                for (int d = 0; d < dI; ++d) {
                    double qd = load_elem(q_idx, q_dtype, (bq * HI + h) * dI + d);
                    double t1 = g * wh * (double)kr[d], t2 = g * wh * qd;
                    dq[(bq * HI + h) * dI + d] += absolute ? fabs(t1) : t1;
                    dk[(b * N + j) * dI + d] += absolute ? fabs(t2) : t2;
                }
            }
        }
    }
    free(kr);
    return OR_OK;
}

/* Gradient of the core attention (oracle_attention) given dout [B][Q][H][D]
 * (float32) for every query row:
 *   dq      [B][Q][H][D]  gradient of the raw query heads,
 *   dkhat_c [B][N][D]     gradient of the prepared compressed rows k_hat
 *                         (what the attention calls read), summed over
 *                         heads and queries,
 *   dkhat_raw [B][R][D]   the same for the prepared window rows,
 *   dsinks [H], dgamma_q [D] (either may be NULL).
 * Per query and head, with do = RoPE_t(dout) (the transpose of the output's
 * rotation by -t), o = sum_u p_u k_u and delta = do . o:
 *   dl_u = p_u (do . k_u - delta),   dz = -p_sink delta,
 *   dq_hat = tau sum_u dl_u k_u,     dk_u += tau dl_u q_hat + p_u do,
 * then dq through RoPE_t's transpose and the RMSNorm of q.  A query with no
 * keys and a -inf sink has zero gradients.  All outputs are overwritten. */
int oracle_attention_bwd(const oracle_attn_params* p, const void* q, const void* kv_c, const int32_t* idx, int K,
                         const void* kv_raw, const int32_t* raw_pos0, const int32_t* q_pos, const float* sinks,
                         const float* gamma_q, const float* gamma_kv, int act_dtype, i64 B, i64 Q, i64 H, i64 D,
                         i64 N, i64 R, const float* dout, double* dq, double* dkhat_c, double* dkhat_raw,
                         double* dsinks, double* dgamma_q) {
    if (p->m < 1 || p->n_win < 0 || p->rope_dims < 0 || (p->rope_dims & 1) || p->rope_dims > D) return OR_EINVAL;
    double tau = p->softmax_scale > 0.0 ? p->softmax_scale : 1.0 / sqrt((double)D);
    memset(dq, 0, sizeof(double) * (size_t)(B * Q * H * D));
    memset(dkhat_c, 0, sizeof(double) * (size_t)(B * N * D));
    memset(dkhat_raw, 0, sizeof(double) * (size_t)(B * R * D));
    if (dsinks) memset(dsinks, 0, sizeof(double) * (size_t)H);
    if (dgamma_q) memset(dgamma_q, 0, sizeof(double) * (size_t)D);
    for (i64 bq = 0; bq < B * Q; ++bq) {
        if (q_pos[bq] < 0) return OR_EINVAL;
        i64 b = bq / Q, t = q_pos[bq];
        i64 nv = n_visible(t, p->m, N);
        i64 ncomp = idx ? K : nv;
        i64 cap = ncomp + p->n_win;
        double* keys = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1) * D);
        double** dst = (double**)malloc(sizeof(double*) * (size_t)(cap > 0 ? cap : 1));
        double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
        i64 nk = 0;
        for (i64 i = 0; i < ncomp; ++i) {
            i64 j = idx ? idx[bq * K + i] : i;
            if (j < 0 || j >= nv) continue;
            for (i64 d = 0; d < D; ++d) tmp[d] = load_elem(kv_c, act_dtype, (b * N + j) * D + d);
            rms_normalise(tmp, gamma_kv, D, p->rms_eps, keys + nk * D);
            rope(keys + nk * D, D, p->rope_dims, p->rope_base, (double)(j * p->m + p->entry_pos_offset));
            dst[nk++] = dkhat_c + (b * N + j) * D;
        }
        i64 p_lo = t - p->n_win + 1;
        if (p_lo < 0) p_lo = 0;
        for (i64 pos = p_lo; pos <= t && p->n_win > 0; ++pos) {
            i64 row = pos - raw_pos0[b];
            if (row < 0 || row >= R) continue;
            for (i64 d = 0; d < D; ++d) tmp[d] = load_elem(kv_raw, act_dtype, (b * R + row) * D + d);
            rms_normalise(tmp, gamma_kv, D, p->rms_eps, keys + nk * D);
            rope(keys + nk * D, D, p->rope_dims, p->rope_base, (double)pos);
            dst[nk++] = dkhat_raw + (b * R + row) * D;
        }
        /* per head: probabilities and logit gradients, then the key rows'
         * gradients summed over heads (rows of one query are distinct) */
        double* P = (double*)malloc(sizeof(double) * (size_t)(H * (nk > 0 ? nk : 1)));
        double* DL = (double*)malloc(sizeof(double) * (size_t)(H * (nk > 0 ? nk : 1)));
        double* QH = (double*)malloc(sizeof(double) * (size_t)(H * D));
        double* DO = (double*)malloc(sizeof(double) * (size_t)(H * D));
        int* live = (int*)malloc(sizeof(int) * (size_t)H);
#pragma omp parallel for schedule(static)
        for (i64 h = 0; h < H; ++h) {
            double* x = (double*)malloc(sizeof(double) * (size_t)D);
            double* u = (double*)malloc(sizeof(double) * (size_t)D);
            double* o = (double*)malloc(sizeof(double) * (size_t)D);
            double* qh = QH + h * D;
            double* doh = DO + h * D;
            for (i64 d = 0; d < D; ++d) x[d] = load_elem(q, act_dtype, (bq * H + h) * D + d);
            rms_normalise(x, gamma_q, D, p->rms_eps, qh);
            rope(qh, D, p->rope_dims, p->rope_base, (double)t);
            double mx = (double)sinks[h];
            for (i64 uu = 0; uu < nk; ++uu) {
                double s = 0.0;
                for (i64 d = 0; d < D; ++d) s += qh[d] * keys[uu * D + d];
                P[h * nk + uu] = tau * s;
                if (P[h * nk + uu] > mx) mx = P[h * nk + uu];
            }
            live[h] = mx != -INFINITY;
            if (!live[h]) {
                for (i64 uu = 0; uu < nk; ++uu) P[h * nk + uu] = DL[h * nk + uu] = 0.0;
                for (i64 d = 0; d < D; ++d) doh[d] = 0.0;
                free(x); free(u); free(o);
                continue;
            }
            double z = exp((double)sinks[h] - mx);
            for (i64 uu = 0; uu < nk; ++uu) {
                P[h * nk + uu] = exp(P[h * nk + uu] - mx);
                z += P[h * nk + uu];
            }
            for (i64 d = 0; d < D; ++d) o[d] = 0.0;
            for (i64 uu = 0; uu < nk; ++uu) {
                P[h * nk + uu] /= z;
                for (i64 d = 0; d < D; ++d) o[d] += P[h * nk + uu] * keys[uu * D + d];
            }
            double psink = exp((double)sinks[h] - mx) / z;
            for (i64 d = 0; d < D; ++d) doh[d] = (double)dout[(bq * H + h) * D + d];
            rope(doh, D, p->rope_dims, p->rope_base, (double)t);
            double delta = 0.0;
            for (i64 d = 0; d < D; ++d) delta += doh[d] * o[d];
            for (i64 d = 0; d < D; ++d) u[d] = 0.0;  /* dq_hat */
            for (i64 uu = 0; uu < nk; ++uu) {
                double dp = 0.0;
                for (i64 d = 0; d < D; ++d) dp += doh[d] * keys[uu * D + d];
                double dl = P[h * nk + uu] * (dp - delta);
                DL[h * nk + uu] = dl;
                for (i64 d = 0; d < D; ++d) u[d] += tau * dl * keys[uu * D + d];
            }
            if (dsinks) {
#pragma omp atomic
                dsinks[h] += -psink * delta;
            }
            /* back through the rotation by t and the RMSNorm of q */
            rope(u, D, p->rope_dims, p->rope_base, -(double)t);
            double* dgq = dgamma_q ? (double*)calloc((size_t)D, sizeof(double)) : NULL;
            rms_normalise_bwd(x, gamma_q, D, p->rms_eps, u, dq + (bq * H + h) * D, dgq);
            if (dgq) {
                for (i64 d = 0; d < D; ++d) {
#pragma omp atomic
                    dgamma_q[d] += dgq[d];
                }
                free(dgq);
            }
            free(x); free(u); free(o);
        }
#pragma omp parallel for schedule(static)
        for (i64 uu = 0; uu < nk; ++uu)
            for (i64 h = 0; h < H; ++h) {
                if (!live[h]) continue;
                for (i64 d = 0; d < D; ++d)
                    dst[uu][d] += tau * DL[h * nk + uu] * QH[h * D + d] + P[h * nk + uu] * DO[h * D + d];
            }
        free(P); free(DL); free(QH); free(DO); free(live);
        free(keys); free(dst); free(tmp);
    }
    return OR_OK;
}
