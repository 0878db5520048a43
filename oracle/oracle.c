/*
 * oracle.c -- plain, slow, fp64 CPU oracle for two-stage GQA block-sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the benchmark's CPU-baseline
 * leg are the only users of this library. The product path (the HIP library) never calls it,
 * and the two share no code: not a header, a helper, a constant or a table.
 *
 * Source of the method: "MiniMax goes sparse: decoding M3's attention from a single diagram"
 * (atlascloud.ai blog; Portuguese, Spanish and French editions; cited below as [MGS]).
 *   [MGS §1, GQA note]   query heads are split into groups; each group shares one K/V set.
 *   [MGS §1, Step 1]     the index branch: one index query per GQA group scores the context;
 *                        token scores are pooled per fixed-size block; TopK keeps the k
 *                        highest-scoring blocks for this layer and this group, giving short
 *                        index lists (one per group).
 *   [MGS §1, Step 2]     the sparse branch: using those lists, the block gathers only the
 *                        selected subsets of the real keys and values and runs attention over
 *                        them; every query head of a group shares the group's selection.
 *   [MGS §2, table and "second subtraction"]  ordinary softmax attention over real K/V, no gate.
 *   [MGS §3]             block size is not given; the post assumes 64 tokens.
 * The formula blocks of the page did not survive extraction, so the steps below are the
 * plainest reading of the prose. Where the page is silent the reading is stated inline:
 *   R1 block summary   = mean of the block's valid keys (the configured "mean-pooled keys");
 *                        a block's score is <index query, summary>, unscaled. By linearity this
 *                        is the mean of the block's token scores.
 *   R2 index query     = mean of the group's query heads (no trained index projection exists).
 *   R3 order           = score descending, then block index ascending; k_eff = min(k, nb);
 *                        the kept list is emitted in ascending block order, padded with -1.
 *   R4 partial block   = the last block of a sequence may hold n_j < P tokens: its summary is
 *                        the mean over those n_j; tokens at or past the length are never read.
 *   R5 decode          = every cached token is visible (the context already holds the current
 *                        token); no forced local or sink block.
 *   R6 prefill         = selection per 64-query tile per group; tile query = mean over the
 *                        tile's rows and the group's heads; candidates = blocks strictly before
 *                        the tile's diagonal block; the diagonal block is always kept and is
 *                        causally masked inside (key position <= query position).
 *   R7 softmax         = logits scale * <q_h, k_t>; weights exp(z - max) / sum; lse = max + ln sum.
 *   R8 index branch    = the page's literal Step 1 (orc_select_index): one index key per token,
 *                        a single head shared by every group (K_idx, dimension d_idx, paged like
 *                        K); one index query per group (given); token score <q_idx[g], K_idx[t]>,
 *                        unscaled; a block's score is the maximum of its valid tokens' scores
 *                        ("Block Max Pool"); then TopK as R3.
 *   R9 forced blocks   = optional, off by default: the first `sink` and the last `local` of a
 *                        row's n candidates are always kept (decode: of the sequence's blocks;
 *                        prefill: of the blocks before the diagonal) and count toward k_eff;
 *                        the other k_eff - |F| come from the remaining candidates under R3.
 *                        The page guesses that an attention sink plus a local block replaced
 *                        NSA's sliding window ([MGS §2], "third subtraction").
 *   R10 bf16 summaries = optional, off by default: the summary pool is stored in bf16; a block
 *                        summary is then its mean (R1) rounded once to the nearest bf16 value,
 *                        ties to even, and every score uses the rounded summary.
 *
 * All arithmetic is fp64 on exact upcasts of the stored inputs (f32 or bf16 bit patterns).
 * Layouts: q [B][Hq][D]; K/V pools [num_pages][Hkv][P][D]; block_table [B][max_blocks].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* R10: x rounded to the nearest value with 8 significant bits (bf16), ties to even; one
 * rounding from the fp64 value. Zero and non-finite values pass through; the means rounded here
 * stay far inside bf16's exponent range. */
static double round_to_bf16(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    double m = frexp(x, &e);                  /* x = m * 2^e, 0.5 <= |m| < 1 */
    return ldexp(rint(ldexp(m, 8)), e - 8);   /* rint: the default mode, nearest-even */
}

/* exact upcast of one stored element */
static double elem(const void* base, int dtype, size_t i) {
    if (dtype == ORC_F32) return (double)((const float*)base)[i];
    uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------ top-k (Step 1, TopK) */
typedef struct { double s; int32_t j; } scored_t;

/* R3: a before b iff s_a > s_b, or equal scores and a has the smaller block index. */
static int by_score_then_index(const void* a, const void* b) {
    const scored_t* x = (const scored_t*)a;
    const scored_t* y = (const scored_t*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

static int ascending_i32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* [MGS §1 Step 1] TopK "keep the k highest-scoring items". Writes k_eff = min(k, n) block
 * indices in ascending order to out[0..k_eff) and -1 to out[k_eff..k). Returns k_eff. */
int orc_topk(const double* s, int n, int k, int32_t* out) {
    if (n < 0 || k < 0) return -1;
    int keff = n < k ? n : k;
    scored_t* v = (scored_t*)malloc(sizeof(scored_t) * (size_t)(n > 0 ? n : 1));
    if (!v) return -1;
    for (int j = 0; j < n; ++j) { v[j].s = s[j]; v[j].j = j; }
    qsort(v, (size_t)n, sizeof(scored_t), by_score_then_index);
    for (int i = 0; i < keff; ++i) out[i] = v[i].j;
    qsort(out, (size_t)keff, sizeof(int32_t), ascending_i32);
    for (int i = keff; i < k; ++i) out[i] = -1;
    free(v);
    return keff;
}

/* R9: forced set F = {j < sink} U {j >= n - local} (of the n candidates), then the best
 * k_eff - |F| of the others under R3; the union in ascending order, padded with -1 to k.
 * Needs sink + local <= k, so that F fits in k_eff = min(k, n). Returns k_eff, or -1. */
int orc_topk_forced(const double* s, int n, int k, int sink, int local, int32_t* out) {
    if (n < 0 || k < 0 || sink < 0 || local < 0 || sink + local > k) return -1;
    int keff = n < k ? n : k;
    char* forced = (char*)calloc((size_t)(n > 0 ? n : 1), 1);
    scored_t* rest = (scored_t*)malloc(sizeof(scored_t) * (size_t)(n > 0 ? n : 1));
    if (!forced || !rest) { free(forced); free(rest); return -1; }
    int nf = 0, m = 0;
    for (int j = 0; j < n; ++j) {
        forced[j] = (char)(j < sink || j >= n - local);
        if (forced[j]) out[nf++] = j;
        else { rest[m].s = s[j]; rest[m].j = j; ++m; }
    }
    qsort(rest, (size_t)m, sizeof(scored_t), by_score_then_index);
    for (int i = 0; i < keff - nf; ++i) out[nf + i] = rest[i].j;
    qsort(out, (size_t)keff, sizeof(int32_t), ascending_i32);
    for (int i = keff; i < k; ++i) out[i] = -1;
    free(forced);
    free(rest);
    return keff;
}

/* ------------------------------------------------------------------ decode */
typedef struct {
    int B, Hq, Hkv, D, P, top_k, keep_sink, keep_local, dtype, num_pages, max_blocks, summary_bf16;
    double scale;
    const void *q, *k_pool, *v_pool;
    const int32_t *block_table, *seq_lens, *idx_in;
    const double* summaries;
    double *scores_out, *o_out, *lse_out, *w_out;
    int32_t* idx_out;
    int status;
} decode_args;

/* element (b, token t, group g, dim d) of a paged pool; -1 if the page id is out of range */
static long long paged_index(const decode_args* a, int b, int t, int g, int d) {
    int32_t page = a->block_table[(size_t)b * a->max_blocks + t / a->P];
    if (page < 0 || page >= a->num_pages) return -1;
    return ((((long long)page * a->Hkv + g) * a->P + (t % a->P)) * a->D + d);
}

/* R1: S_j[g] = (1/n_j) sum of the n_j valid keys of block j, fp64. */
static int block_summary(const decode_args* a, int b, int N, int j, int g, double* S) {
    int t0 = j * a->P;
    int n = N - t0 < a->P ? N - t0 : a->P;
    for (int d = 0; d < a->D; ++d) S[d] = 0.0;
    for (int t = t0; t < t0 + n; ++t)
        for (int d = 0; d < a->D; ++d) {
            long long i = paged_index(a, b, t, g, d);
            if (i < 0) return -1;
            S[d] += elem(a->k_pool, a->dtype, (size_t)i);
        }
    for (int d = 0; d < a->D; ++d) S[d] /= (double)n;
    if (a->summary_bf16)
        for (int d = 0; d < a->D; ++d) S[d] = round_to_bf16(S[d]);
    return 0;
}

/* One (sequence b, KV group g) unit of the decode path: Step 1 then Step 2. */
static int decode_unit(const decode_args* a, int b, int g) {
    const int D = a->D, P = a->P, G = a->Hq / a->Hkv, K = a->top_k;
    int N = a->seq_lens[b];
    if (N < 0) N = 0;
    int nb = (N + P - 1) / P;
    if (nb > a->max_blocks) return -2;
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1));
    double* s = (double*)malloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1));
    double* qidx = (double*)malloc(sizeof(double) * (size_t)D);
    double* S = (double*)malloc(sizeof(double) * (size_t)D);
    if (!sel || !s || !qidx || !S) { free(sel); free(s); free(qidx); free(S); return -3; }
    int rc = 0;

    /* R2: index query = mean of the group's query heads */
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int h = g * G; h < (g + 1) * G; ++h)
            acc += elem(a->q, a->dtype, ((size_t)b * a->Hq + h) * D + d);
        qidx[d] = acc / (double)G;
    }
    /* [MGS §1 Step 1] one score per block: <index query, block summary> (R1) */
    for (int j = 0; j < nb; ++j) {
        const double* Sj = S;
        if (a->summaries) {
            Sj = a->summaries + (((size_t)b * a->max_blocks + j) * a->Hkv + g) * D;
        } else if (block_summary(a, b, N, j, g, S) != 0) { rc = -4; goto done; }
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += qidx[d] * Sj[d];
        s[j] = acc;
    }
    if (a->scores_out) {
        double* row = a->scores_out + ((size_t)b * a->Hkv + g) * a->max_blocks;
        for (int j = 0; j < a->max_blocks; ++j) row[j] = j < nb ? s[j] : -INFINITY;
    }
    /* [MGS §1 Step 1] TopK, or an index list supplied by the caller */
    if (a->idx_in) {
        memcpy(sel, a->idx_in + ((size_t)b * a->Hkv + g) * K, sizeof(int32_t) * (size_t)K);
    } else if (orc_topk_forced(s, nb, K, a->keep_sink, a->keep_local, sel) < 0) { rc = -3; goto done; }
    if (a->idx_out) memcpy(a->idx_out + ((size_t)b * a->Hkv + g) * K, sel, sizeof(int32_t) * (size_t)K);

    /* [MGS §1 Step 2] every head of the group attends over the selected blocks' real K/V */
    for (int h = g * G; h < (g + 1) * G; ++h) {
        double* o = a->o_out + ((size_t)b * a->Hq + h) * D;
        double* w = a->w_out ? a->w_out + ((size_t)b * a->Hq + h) * (size_t)K * P : NULL;
        if (w) for (size_t i = 0; i < (size_t)K * P; ++i) w[i] = 0.0;
        size_t ntok = 0;
        double m = -INFINITY;
        /* pass 1: logits and their max */
        double* z = (double*)malloc(sizeof(double) * (size_t)K * P + 1);
        if (!z) { rc = -3; goto done; }
        for (int e = 0; e < K; ++e) {
            int j = sel[e];
            if (j < 0 || j >= nb) continue;
            int t1 = (j + 1) * P < N ? (j + 1) * P : N;
            for (int t = j * P; t < t1; ++t) {
                double acc = 0.0;
                for (int d = 0; d < D; ++d) {
                    long long i = paged_index(a, b, t, g, d);
                    if (i < 0) { free(z); rc = -4; goto done; }
                    acc += elem(a->q, a->dtype, ((size_t)b * a->Hq + h) * D + d) *
                           elem(a->k_pool, a->dtype, (size_t)i);
                }
                z[ntok] = a->scale * acc;
                if (z[ntok] > m) m = z[ntok];
                ++ntok;
            }
        }
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (ntok == 0) {
            a->lse_out[(size_t)b * a->Hq + h] = -INFINITY;
            free(z);
            continue;
        }
        double den = 0.0;
        for (size_t i = 0; i < ntok; ++i) den += exp(z[i] - m);
        /* pass 2: weights and the weighted sum of values */
        size_t i = 0;
        for (int e = 0; e < K; ++e) {
            int j = sel[e];
            if (j < 0 || j >= nb) continue;
            int t1 = (j + 1) * P < N ? (j + 1) * P : N;
            for (int t = j * P; t < t1; ++t, ++i) {
                double wt = exp(z[i] - m) / den;
                if (w) w[i] = wt;
                for (int d = 0; d < D; ++d)
                    o[d] += wt * elem(a->v_pool, a->dtype, (size_t)paged_index(a, b, t, g, d));
            }
        }
        a->lse_out[(size_t)b * a->Hq + h] = m + log(den);
        free(z);
    }
done:
    free(sel); free(s); free(qidx); free(S);
    return rc;
}

typedef struct { decode_args* a; int tid, nthreads; } decode_job;

static void* decode_worker(void* p) {
    decode_job* job = (decode_job*)p;
    decode_args* a = job->a;
    int units = a->B * a->Hkv;
    for (int u = job->tid; u < units; u += job->nthreads) {
        int rc = decode_unit(a, u / a->Hkv, u % a->Hkv);
        if (rc != 0) a->status = rc;  /* any failure is reported; which one does not matter */
    }
    return NULL;
}

static int run_threads(void* (*fn)(void*), void* jobs, size_t job_size, int nthreads) {
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return -3;
    int started = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, fn, (char*)jobs + job_size * (size_t)i) == 0) started = i;
        else break;
    fn(jobs);  /* thread 0 runs on the caller */
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    free(th);
    return started + 1 == nthreads ? 0 : -5;
}

/* Decode: Step 1 + Step 2 for B sequences, threaded over (b, g) units.
 * summaries (nullable): precomputed [B][max_blocks][Hkv][D] fp64 block summaries, else R1 inline.
 * idx_in (nullable): [B][Hkv][top_k] index lists to attend over instead of selecting
 *   (entries < 0 or >= nb are skipped).
 * scores_out (nullable) [B][Hkv][max_blocks] (-inf past nb), idx_out (nullable) [B][Hkv][top_k],
 * o_out [B][Hq][D], lse_out [B][Hq], w_out (nullable) [B][Hq][top_k*P] weights of the attended
 * tokens in ascending token order, zero-padded.
 * Returns 0, or a negative code (bad argument, page id out of range, allocation failure). */
int orc_decode(int B, int Hq, int Hkv, int D, int P, int top_k, int keep_sink, int keep_local,
               int summary_bf16, double scale, int dtype,
               const void* q, const void* k_pool, const void* v_pool, int num_pages,
               const int32_t* block_table, int max_blocks, const int32_t* seq_lens,
               const double* summaries, const int32_t* idx_in, double* scores_out,
               int32_t* idx_out, double* o_out, double* lse_out, double* w_out, int nthreads) {
    if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || P < 1 || top_k < 1 || !q || !k_pool ||
        !v_pool || !block_table || !seq_lens || !o_out || !lse_out || (dtype != ORC_F32 && dtype != ORC_BF16))
        return -1;
    if (keep_sink < 0 || keep_local < 0 || keep_sink + keep_local > top_k) return -1;
    decode_args a = {B, Hq, Hkv, D, P, top_k, keep_sink, keep_local, dtype, num_pages, max_blocks, summary_bf16 != 0,
                     scale, q, k_pool,
                     v_pool, block_table, seq_lens, idx_in, summaries, scores_out, o_out,
                     lse_out, w_out, idx_out, 0};
    if (nthreads < 1) nthreads = 1;
    decode_job* jobs = (decode_job*)malloc(sizeof(decode_job) * (size_t)nthreads);
    if (!jobs) return -3;
    for (int i = 0; i < nthreads; ++i) { jobs[i].a = &a; jobs[i].tid = i; jobs[i].nthreads = nthreads; }
    int rc = run_threads(decode_worker, jobs, sizeof(decode_job), nthreads);
    free(jobs);
    return a.status ? a.status : rc;
}

/* R1 for every block of every sequence: out [B][max_blocks][Hkv][D] fp64, zero past nb
 * (summary_bf16: each value rounded as R10). */
int orc_summaries(int B, int Hkv, int D, int P, int dtype, int summary_bf16, const void* k_pool, int num_pages,
                  const int32_t* block_table, int max_blocks, const int32_t* seq_lens, double* out) {
    decode_args a;
    memset(&a, 0, sizeof a);
    a.B = B; a.Hq = Hkv; a.Hkv = Hkv; a.D = D; a.P = P; a.dtype = dtype; a.k_pool = k_pool;
    a.num_pages = num_pages; a.block_table = block_table; a.max_blocks = max_blocks;
    a.summary_bf16 = summary_bf16 != 0;
    memset(out, 0, sizeof(double) * (size_t)B * max_blocks * Hkv * D);
    for (int b = 0; b < B; ++b) {
        int N = seq_lens[b] > 0 ? seq_lens[b] : 0;
        int nb = (N + P - 1) / P;
        if (nb > max_blocks) return -2;
        for (int j = 0; j < nb; ++j)
            for (int g = 0; g < Hkv; ++g)
                if (block_summary(&a, b, N, j, g, out + (((size_t)b * max_blocks + j) * Hkv + g) * D))
                    return -4;
    }
    return 0;
}

/* ------------------------------------------------------------------ prefill (R6) */
typedef struct {
    int Hq, Hkv, D, P, top_k, keep_sink, keep_local, summary_bf16, dtype, num_pages, max_blocks, past_len, T,
        tile_lo, tile_hi;
    double scale;
    const void *q, *k_new, *v_new, *k_pool, *v_pool;
    const int32_t* table;        /* one sequence: [max_blocks] */
    const int32_t* idx_in;       /* nullable [ntiles][Hkv][top_k+1] lists to attend over */
    const double* S;             /* [nblocks][Hkv][D] summaries of the appended sequence */
    double *scores_out, *o_out, *lse_out;
    int32_t* idx_out;
    int status;
} prefill_args;

/* key or value element of the sequence after the chunk is appended: cached tokens come from
 * the pool, tokens at positions >= past_len from the chunk. -1 marks a bad page id. */
static int full_elem(const prefill_args* a, int which_v, int t, int g, int d, double* out) {
    if (t >= a->past_len) {
        const void* src = which_v ? a->v_new : a->k_new;
        *out = elem(src, a->dtype, ((size_t)(t - a->past_len) * a->Hkv + g) * a->D + d);
        return 0;
    }
    int32_t page = a->table[t / a->P];
    if (page < 0 || page >= a->num_pages) return -1;
    const void* src = which_v ? a->v_pool : a->k_pool;
    *out = elem(src, a->dtype, ((((size_t)page * a->Hkv + g) * a->P + t % a->P) * a->D + d));
    return 0;
}

static int prefill_unit(const prefill_args* a, int tau, int g) {
    const int D = a->D, P = a->P, G = a->Hq / a->Hkv, K = a->top_k;
    const int i0 = tau * P, i1 = (tau + 1) * P < a->T ? (tau + 1) * P : a->T;
    const int diag = a->past_len / P + tau;        /* the tile's diagonal block */
    double* s = (double*)malloc(sizeof(double) * (size_t)(diag > 0 ? diag : 1));
    double* qt = (double*)malloc(sizeof(double) * (size_t)D);
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K + 1));
    double* z = (double*)malloc(sizeof(double) * (size_t)(K + 1) * P);
    if (!s || !qt || !sel || !z) { free(s); free(qt); free(sel); free(z); return -3; }
    int rc = 0;
    /* tile index query: mean over the tile's rows and the group's heads */
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int i = i0; i < i1; ++i)
            for (int h = g * G; h < (g + 1) * G; ++h)
                acc += elem(a->q, a->dtype, ((size_t)i * a->Hq + h) * D + d);
        qt[d] = acc / (double)((i1 - i0) * G);
    }
    for (int j = 0; j < diag; ++j) {
        const double* Sj = a->S + ((size_t)j * a->Hkv + g) * D;
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += qt[d] * Sj[d];
        s[j] = acc;
    }
    if (a->scores_out) {
        double* row = a->scores_out + ((size_t)tau * a->Hkv + g) * a->max_blocks;
        for (int j = 0; j < a->max_blocks; ++j) row[j] = j < diag ? s[j] : -INFINITY;
    }
    int keff = orc_topk_forced(s, diag, K, a->keep_sink, a->keep_local, sel);
    if (keff < 0) { rc = -3; goto done; }
    sel[keff] = diag;                                  /* the diagonal block is always kept */
    for (int e = keff + 1; e <= K; ++e) sel[e] = -1;
    if (a->idx_out) memcpy(a->idx_out + ((size_t)tau * a->Hkv + g) * (K + 1), sel, sizeof(int32_t) * (size_t)(K + 1));
    if (a->idx_in) {       /* attend over a caller's lists instead (entries < 0 or > diag skipped) */
        memcpy(sel, a->idx_in + ((size_t)tau * a->Hkv + g) * (K + 1), sizeof(int32_t) * (size_t)(K + 1));
        keff = K;
        for (int e = 0; e <= K; ++e) if (sel[e] < 0 || sel[e] > diag) sel[e] = -1;
    }

    for (int i = i0; i < i1; ++i) {
        const int pos = a->past_len + i;
        for (int h = g * G; h < (g + 1) * G; ++h) {
            size_t n = 0;
            double m = -INFINITY, v;
            for (int e = 0; e <= keff; ++e)
                for (int t = sel[e] * P; sel[e] >= 0 && t < (sel[e] + 1) * P && t <= pos; ++t) {
                    double acc = 0.0;
                    for (int d = 0; d < D; ++d) {
                        if (full_elem(a, 0, t, g, d, &v)) { rc = -4; goto done; }
                        acc += elem(a->q, a->dtype, ((size_t)i * a->Hq + h) * D + d) * v;
                    }
                    z[n] = a->scale * acc;
                    if (z[n] > m) m = z[n];
                    ++n;
                }
            double den = 0.0;
            for (size_t r = 0; r < n; ++r) den += exp(z[r] - m);
            double* o = a->o_out + ((size_t)i * a->Hq + h) * D;
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            size_t r = 0;
            for (int e = 0; e <= keff; ++e)
                for (int t = sel[e] * P; sel[e] >= 0 && t < (sel[e] + 1) * P && t <= pos; ++t, ++r) {
                    double wt = exp(z[r] - m) / den;
                    for (int d = 0; d < D; ++d) {
                        if (full_elem(a, 1, t, g, d, &v)) { rc = -4; goto done; }
                        o[d] += wt * v;
                    }
                }
            a->lse_out[(size_t)i * a->Hq + h] = m + log(den);
        }
    }
done:
    free(s); free(qt); free(sel); free(z);
    return rc;
}

typedef struct { prefill_args* a; int tid, nthreads; } prefill_job;

static void* prefill_summary_worker(void* p) {
    prefill_job* job = (prefill_job*)p;
    prefill_args* a = job->a;
    int nblocks = a->past_len / a->P + (a->T + a->P - 1) / a->P;
    double v;
    for (int u = job->tid; u < nblocks * a->Hkv; u += job->nthreads) {
        int j = u / a->Hkv, g = u % a->Hkv;
        double* S = (double*)a->S + ((size_t)j * a->Hkv + g) * a->D;
        int t0 = j * a->P, t1 = (j + 1) * a->P < a->past_len + a->T ? (j + 1) * a->P : a->past_len + a->T;
        for (int d = 0; d < a->D; ++d) S[d] = 0.0;
        for (int t = t0; t < t1; ++t)
            for (int d = 0; d < a->D; ++d) {
                if (full_elem(a, 0, t, g, d, &v)) { a->status = -4; return NULL; }
                S[d] += v;
            }
        for (int d = 0; d < a->D; ++d) S[d] /= (double)(t1 - t0);
        if (a->summary_bf16)
            for (int d = 0; d < a->D; ++d) S[d] = round_to_bf16(S[d]);
    }
    return NULL;
}

static void* prefill_worker(void* p) {
    prefill_job* job = (prefill_job*)p;
    prefill_args* a = job->a;
    int ntile = a->tile_hi - a->tile_lo;
    for (int u = job->tid; u < ntile * a->Hkv; u += job->nthreads) {
        int rc = prefill_unit(a, a->tile_lo + u / a->Hkv, u % a->Hkv);
        if (rc != 0) a->status = rc;
    }
    return NULL;
}

/* Prefill chunk: T new tokens (q, k_new, v_new [T][..][D]) after past_len cached tokens of one
 * sequence (pool + table). Computes tiles [tile_lo, tile_hi) only.
 * idx_in (nullable) [ntiles][Hkv][top_k+1]: lists to attend over instead of the selection.
 * scores_out (nullable) [ntiles][Hkv][max_blocks]; idx_out (nullable) [ntiles][Hkv][top_k+1];
 * o_out [T][Hq][D] and lse_out [T][Hq] (rows of the computed tiles are written). */
int orc_prefill(int Hq, int Hkv, int D, int P, int top_k, int keep_sink, int keep_local, int summary_bf16,
                double scale, int dtype, const void* q, const void* k_new, const void* v_new, const void* k_pool,
                const void* v_pool, int num_pages, const int32_t* table, int max_blocks,
                int past_len, int T, int tile_lo, int tile_hi, const int32_t* idx_in,
                double* scores_out, int32_t* idx_out, double* o_out, double* lse_out, int nthreads) {
    int ntiles = (T + P - 1) / P;
    if (Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || P < 1 || top_k < 0 || T < 1 || past_len < 0 ||
        past_len % P || !q || !k_new || !v_new || !k_pool || !v_pool || !table || !o_out ||
        !lse_out || tile_lo < 0 || tile_hi > ntiles || tile_lo > tile_hi ||
        past_len / P + ntiles > max_blocks || (dtype != ORC_F32 && dtype != ORC_BF16) ||
        keep_sink < 0 || keep_local < 0 || keep_sink + keep_local > top_k)
        return -1;
    int nblocks = past_len / P + ntiles;
    double* S = (double*)malloc(sizeof(double) * (size_t)nblocks * Hkv * D);
    if (!S) return -3;
    prefill_args a = {Hq, Hkv, D, P, top_k, keep_sink, keep_local, summary_bf16 != 0, dtype, num_pages, max_blocks, past_len, T, tile_lo,
                      tile_hi, scale, q, k_new, v_new, k_pool, v_pool, table, idx_in, S,
                      scores_out, o_out, lse_out, idx_out, 0};
    if (nthreads < 1) nthreads = 1;
    prefill_job* jobs = (prefill_job*)malloc(sizeof(prefill_job) * (size_t)nthreads);
    if (!jobs) { free(S); return -3; }
    for (int i = 0; i < nthreads; ++i) { jobs[i].a = &a; jobs[i].tid = i; jobs[i].nthreads = nthreads; }
    int rc = run_threads(prefill_summary_worker, jobs, sizeof(prefill_job), nthreads);
    if (rc == 0 && a.status == 0) rc = run_threads(prefill_worker, jobs, sizeof(prefill_job), nthreads);
    free(jobs);
    free(S);
    return a.status ? a.status : rc;
}

/* ------------------------------------------------------------------ index branch (Step 1, R8) */
/* [MGS §1 Step 1] the index branch as the diagram draws it: per group g, token scores
 * <q_idx[b][g], K_idx[t]> over every valid token t of sequence b, the maximum over each 64-token
 * block (partial last block: its valid tokens), then TopK per (b, g).
 * q_idx [B][Hkv][Di]; ikeys [num_pages][P][Di] (one head), pages through block_table.
 * scores_out (nullable) [B][Hkv][max_blocks] (-inf past the blocks, or for a bad page id);
 * idx_out [B][Hkv][top_k]. Returns 0 on success. */
int orc_select_index(int B, int Hkv, int Di, int P, int top_k, int keep_sink, int keep_local, int dtype,
                     const void* q_idx, const void* ikeys, int num_pages, const int32_t* table, int max_blocks,
                     const int32_t* seq_lens, double* scores_out, int32_t* idx_out) {
    if (B < 0 || Hkv < 1 || Di < 1 || P < 1 || top_k < 0 || !q_idx || !ikeys || !table || !seq_lens ||
        !idx_out || (dtype != ORC_F32 && dtype != ORC_BF16) || keep_sink < 0 || keep_local < 0 ||
        keep_sink + keep_local > top_k)
        return -1;
    double* row = (double*)malloc(sizeof(double) * (size_t)(max_blocks > 0 ? max_blocks : 1));
    if (!row) return -3;
    for (int b = 0; b < B; ++b) {
        int N = seq_lens[b];
        if (N < 0 || N > max_blocks * P) { free(row); return -2; }
        int nb = (N + P - 1) / P;
        for (int g = 0; g < Hkv; ++g) {
            for (int j = 0; j < nb; ++j) {
                int32_t page = table[(size_t)b * max_blocks + j];
                double best = -INFINITY;
                if (page >= 0 && page < num_pages) {
                    int n_j = N - j * P < P ? N - j * P : P;
                    for (int t = 0; t < n_j; ++t) {
                        double s = 0.0;
                        for (int d = 0; d < Di; ++d)
                            s += elem(q_idx, dtype, ((size_t)b * Hkv + g) * Di + d) *
                                 elem(ikeys, dtype, ((size_t)page * P + t) * Di + d);
                        if (s > best) best = s;
                    }
                }
                row[j] = best;
            }
            if (scores_out) {
                double* srow = scores_out + ((size_t)b * Hkv + g) * max_blocks;
                for (int j = 0; j < max_blocks; ++j) srow[j] = j < nb ? row[j] : -INFINITY;
            }
            if (orc_topk_forced(row, nb, top_k, keep_sink, keep_local, idx_out + ((size_t)b * Hkv + g) * top_k) < 0) {
                free(row);
                return -3;
            }
        }
    }
    free(row);
    return 0;
}
